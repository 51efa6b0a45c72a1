/*
 * routed_moe.h -- C ABI of the MI355X (gfx950) routed Mixture-of-Experts layer.
 *
 * The layer ("Cake SiTU backend", FlashInfer docs, intro paragraph): BF16 tokens x[T,H]
 * are quantized to group-16 NVFP4, routed to top-k experts, pushed through FC1 (fused
 * gate/up rows), the SiTU activation, NVFP4 requantization and FC2, and combined with
 * the BF16 route weights into BF16 out[T,H].  The routing primitive follows
 * "torch_npu.npu_moe_init_routing_v2" (Ascend API reference, section 计算公式).
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are GPU global-memory addresses; "host" are CPU memory.
 *     The caller owns every buffer; the library never allocates, frees or retains one.
 *   - Work is enqueued on `stream` (0 = the null stream) and runs asynchronously; the
 *     library never reads device memory back to the host and never synchronizes, so a
 *     whole call can be captured into a hipGraph and replayed ("Cake SiTU backend",
 *     section "Caller-owned execution": submission allocates nothing and owns no graph).
 *   - Arguments are validated on the host before any HIP call; a bad argument returns
 *     an error code and enqueues nothing.  Device-side data (expert ids, scales) is
 *     the caller's contract and is not checked (ids must lie in [0, E)).
 *   - Calls that run concurrently need distinct workspace and output buffers.
 *   - BF16 is passed as 16-bit patterns; "E4M3" is float8_e4m3fn (bias 7, max 448);
 *     NVFP4 codes are E2M1 nibbles, two per byte, element 2b in the low nibble of byte b.
 */
#ifndef ROUTED_MOE_H
#define ROUTED_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* moe_stream_t;   /* a hipStream_t */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,        /* null/misaligned pointer, size out of range */
  MOE_ERR_UNSUPPORTED = -2,        /* dimensions outside what the kernels implement */
  MOE_ERR_WORKSPACE_TOO_SMALL = -3,
  MOE_ERR_HIP = -4                 /* a HIP launch or runtime call failed */
} moe_status_t;

/* Layer dimensions: H (hidden), I (intermediate, per TP rank), E (experts), k (top-k).
 * Supported: H % 128 == 0, I % 64 == 0, 128 <= H <= 16384, 64 <= I <= 4096,
 * 1 <= E <= 4096, 1 <= k <= 64.  The page's shape is H=3584, I=384, E=896, k=16
 * ("Cake SiTU backend", intro). */
typedef struct {
  int32_t hidden;
  int32_t inter;
  int32_t num_experts;
  int32_t top_k;
} moe_dims_t;

/* Largest token count of one moe_forward call ("Cake SiTU backend", intro: 1..16384). */
#define MOE_MAX_TOKENS 16384

/* Quantization of the tokens a call moves or computes on:
 *   MOE_QUANT_NONE             BF16 as given;
 *   MOE_QUANT_INT8_ROW_DYNAMIC per-row dynamic int8 ("torch_npu.npu_moe_init_routing_v2",
 *                              section 计算公式 step 4: scale = row_max|x| / 127);
 *   MOE_QUANT_NVFP4_G16        group-16 NVFP4 with the global encoding scale qx, the
 *                              layer's input quantization ("Cake SiTU backend", intro; the
 *                              arithmetic is given at moe_quantize_nvfp4). */
typedef enum {
  MOE_QUANT_NONE = 0,
  MOE_QUANT_INT8_ROW_DYNAMIC = 1,
  MOE_QUANT_NVFP4_G16 = 2
} moe_quant_t;

/* Human-readable text of a status code (static storage; never NULL). */
const char* moe_status_string(moe_status_t s);

/* ------------------------------------------------------------------------------------
 * Sizes.  Host-only: no HIP call, no device access ("Cake SiTU backend", section
 * "Caller-owned execution": the size query uses host metadata only).
 * ------------------------------------------------------------------------------------ */

/* Workspace bytes for every T <= max_tokens of moe_route with quantization q and, when q
 * is MOE_QUANT_NVFP4_G16 (the layer's quantization), of moe_forward too; the layer's
 * limits on d and T (<= MOE_MAX_TOKENS) then apply.  moe_route reads only d.hidden,
 * d.num_experts and d.top_k.  Monotone in max_tokens, so a buffer sized for the maximum
 * serves every smaller call (same section). */
moe_status_t moe_workspace_size(moe_dims_t d, int32_t max_tokens, moe_quant_t q,
                                size_t* bytes /*host*/);

/* Bytes of the prepared (re-laid-out) weights written by moe_prepare_weights: the FC1 and
 * FC2 codes and block scales, E * (2I*H/2 + 2I*H/16 + H*Ip/2 + H*Ip/16) with Ip = I
 * rounded up to a multiple of 128 (zero padding). */
moe_status_t moe_prepared_weights_size(moe_dims_t d, size_t* bytes /*host*/);

/* Byte offsets, inside the moe_forward workspace for a call with T tokens, of the
 * intermediates that call leaves behind (for inspection and testing; the contents are
 * valid after the call completes and until the workspace is reused):
 *   x_codes   u8  [T, H/2]    NVFP4 codes of x           x_scales  u8  [T, H/16] E4M3
 *   x_dec     f16 [T, H]      x's NVFP4 values before the global scale (code times block
 *                             scale, exact in f16): the FC1 operand; written only when
 *                             T*k < 2 * 128 * (compute units of the device), 65536 on
 *                             an MI355X (with more routed rows FC1 stages the codes and
 *                             this region is left as it was)
 *   sorted_ids      i32 [T*k] expert of each sorted row  (keyValueSort keys)
 *   sorted_row_idx  i32 [T*k] flat id t*k+j of each sorted row
 *   expanded_row_idx i32 [T*k] gather map: sorted position of flat id f
 *   expert_counts   i32 [E]   rows per expert;  expert_cumsum i32 [E] inclusive prefix sum
 *   a_codes   u8  [T*k, I/2]  requantized SiTU output, sorted row order
 *   a_scales  u8  [T*k, I/16]
 *   o_rows    f16  [T*k, H]   FC2 output O of routed row (t, j) at row t*k + j, alpha2
 *                             applied, stored as O * 2^s (rows of dropped ids are not
 *                             written)
 *   o_exp     i8   [T*k]      s of routed row t*k + j: one exponent per expert e, from a
 *                             bound (|FC2 sum| <= I * 2688^2): with E the fp32 biased
 *                             exponent of |alpha2[e]| * I * 2688^2, s = clamp(141 - E,
 *                             -126, 126), so every |O| * 2^s is below 2^15
 *   a_amax    f32 [E]         max |SiTU output| of each expert's rows in this call
 *                             (0 for an expert with no rows; a calibration statistic) */
typedef struct {
  size_t x_codes, x_scales, x_dec;
  size_t sorted_ids, sorted_row_idx, expanded_row_idx;
  size_t expert_counts, expert_cumsum;
  size_t a_codes, a_scales;
  size_t o_rows, o_exp;
  size_t a_amax;
  size_t total;              /* bytes the call uses; <= moe_workspace_size(T) */
} moe_workspace_layout_t;

moe_status_t moe_workspace_layout(moe_dims_t d, int32_t T, moe_workspace_layout_t* out /*host*/);

/* Workspace bytes of moe_route and moe_route_v2 for num_rows tokens, top_k, num_experts
 * (moe_workspace_size with q other than MOE_QUANT_NVFP4_G16 returns the same). */
moe_status_t moe_route_workspace_size(int32_t num_rows, int32_t top_k, int32_t num_experts,
                                      size_t* bytes /*host*/);

/* ------------------------------------------------------------------------------------
 * Preparation (once, before any forward call).
 * ------------------------------------------------------------------------------------ */

/* Group-16 NVFP4 quantization of BF16 rows with one fp32 encoding scale per group of
 * rows: src is [groups, rows_per_group, K] BF16 (device, contiguous); q is float32
 * [groups] (device); codes u8 [groups*rows_per_group, K/2], scales u8 [.., K/16] (device).
 * Per 16 consecutive values v of a row: s = E4M3(min(fp32(fp32(amax|v| * q)/6), 448)),
 * round-to-nearest-even; enc = q/s (0 when s = 0); code = E2M1(fp32(v*enc)),
 * nearest-even, saturating at 6, sign kept.  This is the "group-16 NVFP4 input
 * quantization" of "Cake SiTU backend" (intro; the scale arithmetic order is this
 * library's reading, the pages do not give it).  Used for x inside moe_forward and for
 * weights (one group per expert, q = qW[e]) at preparation.  K % 16 == 0, K <= 65536. */
moe_status_t moe_quantize_nvfp4(const uint16_t* src /*device*/, int64_t groups,
                                int64_t rows_per_group, int32_t K, const float* q /*device*/,
                                uint8_t* codes /*device*/, uint8_t* scales /*device*/,
                                moe_stream_t stream);

/* Re-lay canonical NVFP4 expert weights into the library's private layout ("Cake SiTU
 * backend", section "Prepared weights and scales": weights are prepared once and their
 * block scales travel with the packed bytes).  Canonical inputs (device, contiguous):
 *   w13 u8 [E, 2I, H/2]  FC1 codes, rows [0,I) gate then [I,2I) up;  w13_sf u8 [E, 2I, H/16]
 *   w2  u8 [E, H, I/2]   FC2 codes;                                   w2_sf  u8 [E, H, I/16]
 * `prepared` (device) receives moe_prepared_weights_size() bytes; it must not alias the
 * inputs.  The layout is private: only moe_forward reads it. */
moe_status_t moe_prepare_weights(moe_dims_t d, const uint8_t* w13, const uint8_t* w13_sf,
                                 const uint8_t* w2, const uint8_t* w2_sf, void* prepared,
                                 size_t prepared_bytes, moe_stream_t stream);

/* ------------------------------------------------------------------------------------
 * The routing primitive ("torch_npu.npu_moe_init_routing_v2", section 计算公式, steps
 * 1-5, dropless, full expert range, gather index type 0, cumsum histogram type 0), with
 * the token movement quantized as q:
 *   sorted_expert_ids, sorted_row_idx = stable keyValueSort(expert_ids, f = t*k + j)
 *   expanded_row_idx[sorted_row_idx[i]] = i
 *   expert_cumsum[e] = number of rows with expert <= e          (inclusive)
 *   q MOE_QUANT_NONE:             expanded_x[i] = x[sorted_row_idx[i] / k]  (BF16 [T*k, H])
 *   q MOE_QUANT_INT8_ROW_DYNAMIC: scale_t = fp32(row_max|x_t| / 127),
 *        q_t = clip(round_half_even(fp32(x_t / scale_t)), -127, 127) (0 if scale_t == 0),
 *        expanded_x[i] = q_{sorted_row_idx[i]/k} (int8 [T*k, H]),
 *        expanded_sf_or_scale[i] = scale_t (f32 [T*k]);
 *   q MOE_QUANT_NVFP4_G16:        token t quantized as moe_quantize_nvfp4 with q = *qx,
 *        expanded_x[i] = its codes (u8 [T*k, H/2]), expanded_sf_or_scale[i] = its E4M3
 *        block scales (u8 [T*k, H/16]), t = sorted_row_idx[i] / k (one read of each token,
 *        one quantization, its k rows written).
 * Buffers (device): x BF16 [T, H]; expert_ids i32 [T, k] with values in [0, E);
 * qx f32 [1] (NVFP4 only, else may be NULL); expanded_sf_or_scale NULL for MOE_QUANT_NONE;
 * expanded_row_idx, sorted_expert_ids, sorted_row_idx i32 [T*k] (the last two may be
 * NULL); expert_cumsum i32 [E].  d.inter is not used.  Limits: 1 <= T, T*k <= 2^24,
 * H % 8 == 0 (H % 16 == 0 for NVFP4), H <= 65536, 1 <= E <= 10240 (the page's expert_num
 * limit), 1 <= k <= 64.
 * workspace: moe_workspace_size(d, T, q) bytes, 256-byte aligned.
 * ------------------------------------------------------------------------------------ */
moe_status_t moe_route(moe_dims_t d, int32_t T, const uint16_t* x, const int32_t* expert_ids,
                       moe_quant_t q, const float* qx, int32_t* sorted_expert_ids,
                       int32_t* sorted_row_idx, int32_t* expanded_row_idx,
                       int32_t* expert_cumsum, void* expanded_x, void* expanded_sf_or_scale,
                       void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* ------------------------------------------------------------------------------------
 * The routing primitive with the options of the same page ("torch_npu.
 * npu_moe_init_routing_v2": section 计算公式 steps 1-6 and the parameter list).
 *
 *   expert_start, expert_end  active expert range [start, end) (0, 0 = all experts).
 *        Ids outside it take no part: the in-range ids, stably sorted, occupy positions
 *        0 .. avail-1, avail = availableIdxNum = the number of in-range ids (step 6).
 *   row_idx_type  0: expanded_row_idx[f] = position of flat id f (gather index), -1 for
 *        an out-of-range id;  1: expanded_row_idx[i] = flat id at position i (scatter
 *        index), -1 for i >= avail (the page leaves those unwritten).
 *   expert_tokens_num_type  (step 3, over the range, counting every in-range id)
 *        0: inclusive cumsum [end-start];  1: per-expert count [end-start];
 *        2: key_value [num_experts, 2] = (expert id, count) of the in-range experts with
 *        a nonzero count, increasing id, then rows of 0.
 *   quant_mode  -1: BF16 copy (with a per-row scale [N] given as `scale`, expanded_scale
 *        [i] = scale[row of i]);  0: static int8, q = clip(round_half_even(fp32(fp32(
 *        x * scale[0]) + offset[0])), -128, 127), no expanded_scale;  1: dynamic int8
 *        exactly as moe_route (expanded_scale required).
 *   drop_pad_mode 1 with expert_capacity C (1 <= C <= N*K; needs the full range, the
 *        gather index and active_num <= 0): expanded_x is [num_experts, C, H]; expert e's
 *        rows in sorted order fill slots e*C + r for r < C, later rows are dropped
 *        (expanded_row_idx -1), empty slots are 0 (expanded_scale 0).
 *   active_num  > 0: only expanded rows 0 .. active_num-1 exist (expanded_x is
 *        [min(active_num, N*K), H]); <= 0: no limit.  Index outputs are unaffected.
 *
 * Buffers (device): x BF16 [N, H]; expert_idx i32 [N, K] with values in [0, num_experts);
 * scale, offset f32 as above (else NULL); expanded_x as above (BF16 or int8; rows past
 * the valid ones are left untouched except drop/pad's zero slots); expanded_row_idx i32
 * [N*K]; expert_tokens i32 as above or NULL; expanded_scale f32 [rows of expanded_x] or
 * NULL; available_idx_num i32 [1] or NULL.  workspace: moe_route_workspace_size() bytes.
 * Limits as moe_route: num_experts <= 10240, and <= 5120 with the key_value histogram
 * (the page's expert_num limits).  The smoothing-scale variant of the dynamic mode is
 * not offered.
 * ------------------------------------------------------------------------------------ */
typedef struct {
  int32_t expert_start;
  int32_t expert_end;
  int32_t row_idx_type;
  int32_t expert_tokens_num_type;
  int32_t quant_mode;
  int32_t drop_pad_mode;
  int32_t expert_capacity;
  int32_t active_num;
} moe_route_options_t;

moe_status_t moe_route_v2(int32_t num_rows, int32_t hidden, int32_t num_experts, int32_t top_k,
                          const uint16_t* x, const int32_t* expert_idx, const float* scale,
                          const float* offset, const moe_route_options_t* opts /*host*/,
                          void* expanded_x, int32_t* expanded_row_idx, int32_t* expert_tokens,
                          float* expanded_scale, int32_t* available_idx_num, void* workspace,
                          size_t workspace_bytes, moe_stream_t stream);

/* ------------------------------------------------------------------------------------
 * The whole layer ("Cake SiTU backend": intro for the stages; section "Prepared weights
 * and scales" for the scales and SiTU; "Caller-owned execution" for the contract).
 *   x              BF16 [T, H]            (device)
 *   expert_ids     i32  [T, k]  in [0,E)  (device)
 *   route_weights  BF16 [T, k]            (device; used as given, not renormalized)
 *   prepared       moe_prepare_weights output (device)
 *   qx             f32 [1]  activation encoding scale qX = 1/dX          (device)
 *   alpha1         f32 [E]  FC1 dequantization dX*dW13[e]                (device)
 *   qa             f32 [E]  intermediate encoding scale qA[e] = 1/dA[e]  (device)
 *   alpha2         f32 [E]  FC2 dequantization dA[e]*dW2[e]              (device)
 *   situ_beta      f32 [E] or NULL (then 4)   gate smoothing beta        (device)
 *   situ_linear_beta f32 [E] or NULL (then 25) linear smoothing lambda   (device)
 *   workspace      >= moe_workspace_size(d, T) bytes, 256-byte aligned   (device)
 *   out            BF16 [T, H]                                            (device)
 * SiTU(g, u) = (beta*tanh(g/beta)*sigmoid(g)) * (lambda*tanh(u/lambda)) with g the FC1
 * gate row and u the matching up row.  out[t] = BF16(sum_j w[t,j] * O[t,j]) with O the
 * FC2 output of (t, j) and the sum in j order in fp32.  1 <= T <= MOE_MAX_TOKENS.
 * ------------------------------------------------------------------------------------ */
moe_status_t moe_forward(moe_dims_t d, int32_t T, const uint16_t* x, const int32_t* expert_ids,
                         const uint16_t* route_weights, const void* prepared, const float* qx,
                         const float* alpha1, const float* qa, const float* alpha2,
                         const float* situ_beta, const float* situ_linear_beta,
                         void* workspace, size_t workspace_bytes, uint16_t* out,
                         moe_stream_t stream);

/* moe_forward with per-stage timing events, for profiling.  The work and its results are
 * identical to moe_forward.  `events` is a host array of MOE_FORWARD_STAGES + 1 hipEvent_t
 * handles created by the caller; event i is recorded on `stream` at the start of stage i
 * and event MOE_FORWARD_STAGES after the last stage.  The stages are, in order: 0 NVFP4
 * quantization of x, 1 routing (histogram, scan, scatter), 2 FC1 + SiTU + requantization,
 * 3 FC2, 4 finalization.  With at most 1024 routed rows (T*k) and E <= 3276 the
 * quantization and the routing run as one launch; events 1 and 2 are then both recorded
 * after it, so stage 0 holds both and stage 1 is empty.  The caller reads the stage durations with
 * hipEventElapsedTime once the events have completed.  NULL events -> MOE_ERR_INVALID_ARG. */
#define MOE_FORWARD_STAGES 5
moe_status_t moe_forward_timed(moe_dims_t d, int32_t T, const uint16_t* x,
                               const int32_t* expert_ids, const uint16_t* route_weights,
                               const void* prepared, const float* qx, const float* alpha1,
                               const float* qa, const float* alpha2, const float* situ_beta,
                               const float* situ_linear_beta, void* workspace,
                               size_t workspace_bytes, uint16_t* out, moe_stream_t stream,
                               void* const* events);

/* ------------------------------------------------------------------------------------
 * moe_forward for callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid allocation): the same computation and
 * arguments without `workspace`, using instead a fixed array of MOE_NOALLOC_SCRATCH_BYTES
 * in each GPU's global memory that the library holds until the process ends (its device
 * address is looked up on the first call on a device).  The call itself allocates nothing.
 * Sizes whose workspace (moe_workspace_size(d, T, MOE_QUANT_NVFP4_G16)) exceeds the array
 * return MOE_ERR_UNSUPPORTED: at the page's shape that is T > 262.  Every call on one GPU
 * uses that GPU's one array, so calls on one GPU must not overlap (on different streams
 * they race); the array keeps the last call's intermediates.
 * ------------------------------------------------------------------------------------ */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

moe_status_t moe_forward_noalloc(moe_dims_t d, int32_t T, const uint16_t* x,
                                 const int32_t* expert_ids, const uint16_t* route_weights,
                                 const void* prepared, const float* qx, const float* alpha1,
                                 const float* qa, const float* alpha2, const float* situ_beta,
                                 const float* situ_linear_beta, uint16_t* out,
                                 moe_stream_t stream);

/* ------------------------------------------------------------------------------------
 * The step before the layer: top-k expert selection with softmax route weights.  The
 * layer takes expert ids and BF16 route weights as given ("Cake SiTU backend", intro);
 * the pages do not define the gate that makes the router logits, so they are an input:
 *   expert_ids[t, 0..k-1] = the k largest logits of token t in decreasing order (equal
 *       logits in increasing expert id);
 *   route_weights[t, j] = BF16(exp(l_j - l_0) / sum_i exp(l_i - l_0)) over those k logits
 *       (fp32 arithmetic, round to nearest even).
 * Buffers (device): logits f32 [T, num_experts] (finite values), expert_ids i32 [T, k],
 * route_weights BF16 [T, k] -- the layout moe_forward takes.  Limits: 1 <= T,
 * 1 <= num_experts <= 4096, 1 <= top_k <= min(num_experts, 64).
 * ------------------------------------------------------------------------------------ */
moe_status_t moe_topk_softmax(int32_t T, int32_t num_experts, int32_t top_k,
                              const float* logits, int32_t* expert_ids, uint16_t* route_weights,
                              moe_stream_t stream);

/* ------------------------------------------------------------------------------------
 * Chunk-streamed front end, one rank ("[RFC] Chunk-ready symmetric-buffer protocol for
 * streaming MegaMoE inputs": sections "Fixed-capacity ring", "Independent readiness
 * generations", "Memory ordering", "Chunk-aware dispatch scheduling" options 1 --
 * chunk-local expert pools, moe_forward_streamed -- and 2 -- reservations across chunks
 * with an end-of-stream seal, moe_forward_absorb + moe_forward_seal -- and "Progress and
 * deadlock requirements").
 *
 * A caller-owned ring of num_slots slots of tokens_per_slot (C) tokens.  Token chunk n
 * (tokens n*C .. min((n+1)*C, total) - 1) lives in slot n % num_slots.  Two producers fill
 * a slot independently, in either order: the ROUTE producer writes expert_ids [C, k] i32
 * and route_weights [C, k] BF16, the LAYOUT producer writes x [C, H] BF16.  Each producer,
 * for each chunk, on its own stream:
 *     moe_ring_acquire(slot, role)   -- waits until the consumer has finished the slot's
 *                                       previous contents from this producer
 *     ... write the payload part (kernels or copies on the same stream) ...
 *     moe_ring_publish(slot, role)   -- publishes the next generation of its part
 * moe_forward_streamed consumes chunks in order: it waits for both parts of a chunk, runs
 * the whole layer on that chunk alone (its own routing and expert tiles) into out rows
 * n*C .., and publishes the slot as consumed.  Generations are per slot and per role and
 * count uses of the slot; all sequence counters live in the ring, so a launch sequence
 * captured into a graph stays valid over any number of replays.  Publishes are
 * system-scope release stores after the payload writes that precede them on the stream;
 * waits are system-scope acquire loads.
 *
 * Progress: every wait is a one-workgroup kernel bounded by timeout_us (0 = 1 s).  When
 * a wait expires it records MOE_RING_CONSUMER_TIMEOUT or MOE_RING_PRODUCER_TIMEOUT in the
 * ring's status word (the first failure is kept) and returns.  While the status word holds
 * a failure, the consumer takes no expert id from a slot: every chunk it consumes or
 * absorbs has all its ids dropped, so its output rows are zero (a defined value, never
 * computed from stale slot data), and the slot is still published as consumed.  The ring
 * must then be re-initialized.  The rule for progress:
 * enqueue every publish before the waits that need it (in host enqueue order, across
 * streams), for example all chunks produced into a ring of at least as many slots and
 * then consumed, or produce and consume alternating per chunk.  Then any placement of the
 * streams works: streams on different hardware queues overlap, and streams the runtime
 * puts on one hardware queue run in enqueue order.  A wait enqueued before a publish it
 * needs can make progress only if the runtime runs the two streams on different hardware
 * queues; otherwise it expires.
 * ------------------------------------------------------------------------------------ */
typedef enum { MOE_RING_ROUTE = 0, MOE_RING_LAYOUT = 1 } moe_ring_role_t;

/* Values of the ring's status word (u32 at moe_ring_layout_t.status). */
#define MOE_RING_OK 0u
#define MOE_RING_CONSUMER_TIMEOUT 1u
#define MOE_RING_PRODUCER_TIMEOUT 2u

typedef struct {
  void* base;               /* device, 256-byte aligned */
  size_t bytes;             /* >= moe_ring_layout().total */
  int32_t num_slots;        /* 1 .. 4096 */
  int32_t tokens_per_slot;  /* 1 .. MOE_MAX_TOKENS */
} moe_ring_t;

/* Byte offsets inside the ring (host-only):
 *   x              BF16 [num_slots, C, H]
 *   expert_ids     i32  [num_slots, C, k]
 *   route_weights  BF16 [num_slots, C, k]
 *   counters       one 64-byte record per slot: u32 route_ready_gen, layout_ready_gen,
 *                  consumed_gen, then the three owners' private sequences
 *   status         u32 */
typedef struct {
  size_t x, expert_ids, route_weights, counters, status, total;
} moe_ring_layout_t;

moe_status_t moe_ring_layout(moe_dims_t d, int32_t num_slots, int32_t tokens_per_slot,
                             moe_ring_layout_t* out /*host*/);

/* Zero the counters and the status word (a kernel on `stream`, no memset). */
moe_status_t moe_ring_init(moe_dims_t d, const moe_ring_t* ring /*host*/, moe_stream_t stream);

moe_status_t moe_ring_acquire(moe_dims_t d, const moe_ring_t* ring /*host*/, int32_t slot,
                              moe_ring_role_t role, uint32_t timeout_us, moe_stream_t stream);

moe_status_t moe_ring_publish(moe_dims_t d, const moe_ring_t* ring /*host*/, int32_t slot,
                              moe_ring_role_t role, moe_stream_t stream);

/* The layer (as moe_forward) over chunks first_chunk .. first_chunk + num_chunks - 1 of a
 * stream of total_tokens tokens; out is BF16 [total_tokens, H] (device) and receives the
 * rows of those chunks.  workspace: moe_workspace_size(d, tokens_per_slot) bytes. */
moe_status_t moe_forward_streamed(moe_dims_t d, const moe_ring_t* ring /*host*/,
                                  int32_t total_tokens, int32_t first_chunk,
                                  int32_t num_chunks, const void* prepared, const float* qx,
                                  const float* alpha1, const float* qa, const float* alpha2,
                                  const float* situ_beta, const float* situ_linear_beta,
                                  uint32_t timeout_us, void* workspace, size_t workspace_bytes,
                                  uint16_t* out, moe_stream_t stream);

/* Scheduling option 2 of the same RFC section, with the completion rule that every expert
 * block is complete at the end-of-stream seal: the stream's routed rows are packed per
 * expert over all its chunks, as in one moe_forward over the whole stream.
 *
 * moe_forward_absorb consumes chunks first_chunk .. first_chunk + num_chunks - 1 of a
 * stream of total_tokens tokens in order, like moe_forward_streamed: for each it waits for
 * both parts, quantizes the chunk's tokens (qx as in moe_forward) into the stream's rows of
 * the workspace, copies its expert ids and route weights there, and publishes the slot as
 * consumed, so the slot can be refilled before the stream ends.  Absorb the chunks in
 * stream order, each once, in any number of calls (for example one call per chunk,
 * alternating with the producers, under the progress rule above).
 *
 * moe_forward_seal then runs the routing, FC1, SiTU, requantization, FC2 and the
 * finalization once over all total_tokens tokens into out, BF16 [total_tokens, H]; the
 * result equals moe_forward on the whole stream bit for bit.
 *
 * workspace: moe_sealed_workspace_size(d, total_tokens) bytes, 256-byte aligned (device),
 * the same buffer and the same total_tokens for every absorb call and the seal of one
 * stream; every chunk of the stream must be absorbed before the seal.  Its first
 * moe_workspace_size(d, total_tokens) bytes hold moe_forward's workspace layout for
 * total_tokens tokens (moe_workspace_layout) after the seal. */
moe_status_t moe_sealed_workspace_size(moe_dims_t d, int32_t total_tokens,
                                       size_t* bytes /*host*/);

moe_status_t moe_forward_absorb(moe_dims_t d, const moe_ring_t* ring /*host*/,
                                int32_t total_tokens, int32_t first_chunk, int32_t num_chunks,
                                const float* qx, uint32_t timeout_us, void* workspace,
                                size_t workspace_bytes, moe_stream_t stream);

moe_status_t moe_forward_seal(moe_dims_t d, int32_t total_tokens, const void* prepared,
                              const float* alpha1, const float* qa, const float* alpha2,
                              const float* situ_beta, const float* situ_linear_beta,
                              void* workspace, size_t workspace_bytes, uint16_t* out,
                              moe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ROUTED_MOE_H */
