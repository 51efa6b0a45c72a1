// Grouped GEMMs of the routed MoE layer on the f16 MFMA (16x16x32, fp32 accumulate) and
// the BF16 weighted finalization.
//
// "Cake SiTU backend" (intro; section "Prepared weights and scales"):
//   FC1: h[r, n] = alpha1[e] * sum_k xhat[r, k] * w13hat[e, n, k]    n in [0, 2I)
//   SiTU: a = (beta*tanh(g/beta)*sigmoid(g)) * (lambda*tanh(u/lambda)), g = h[.., i],
//         u = h[.., I + i]; then group-16 NVFP4 requantization with qA[e]
//   FC2: o[r, h] = alpha2[e] * sum_i ahat[r, i] * w2hat[e, h, i]
//   out[t] = BF16(sum_j w[t, j] * o[row(t, j)])
// where xhat, what, ahat are NVFP4 values decoded exactly (E2M1 code times E4M3 block
// scale: at most 6 significant bits, so exact in f16), and alpha multiplies the fp32
// accumulator after block dequantization ("Nvfp4 Tensor": the global scale is applied
// after block dequantization).
//
// Work decomposition: the router writes two lists of token tiles (expert-sorted rows of
// one expert): "small" tiles of up to 32 rows (one per lightly used expert) and "big" tiles
// of up to 128 rows.  Each list has its own kernel instance.  A workgroup (4 waves) takes
// one token tile and a slab of weight rows; each wave owns WRG 16-row MFMA groups of the
// slab and all tokens of the tile:
//   * weights stream from HBM straight into registers in the prepared layout (one 16-byte
//     load per lane per group per 128-column chunk), one chunk ahead of the MFMAs, and are
//     decoded to f16 in registers (each wave owns its rows, so nothing is decoded twice);
//   * the token tile's codes for the next chunk are loaded into registers, decoded once per
//     workgroup to f16 and written to a double-buffered LDS tile that all four waves read
//     as MFMA operands (one barrier per chunk).
// The FC1 epilogue fuses alpha1, SiTU, the group-16 requantization (two consecutive MFMA
// row groups hold the gate/up pairs of 16 intermediate channels = one NVFP4 group) and the
// per-expert amax statistic; the FC2 epilogue applies alpha2 and stores the rows as f16
// scaled by a power of two per expert (store_out_block).
#include <type_traits>

#include "common.h"
#include "fc2_tile.h"
#include "gemm_util.h"
#include "kernels.h"

namespace rmoe {

// SiTU(g, u) = (beta*tanh(g/beta)*sigmoid(g)) * (lam*tanh(u/lam)), written with
// exponentials of non-positive arguments only (no overflow) and one reciprocal:
//   tanh(x) = sign(x) (1 - t)/(1 + t), t = exp(-2|x|);
//   sigmoid(g) = (g >= 0 ? 1 : s)/(1 + s), s = exp(-|g|);
// so SiTU = beta*lam*sign(g u) (1-t1)(1-t2)(g>=0 ? 1 : s) / ((1+t1)(1+t2)(1+s)), every
// denominator factor in [1, 2].  exp uses the hardware base-2 exponential.
__device__ __forceinline__ float situ(float g, float u, float beta, float inv_beta,
                                      float lam, float inv_lam) {
  constexpr float kLog2e = 1.4426950408889634f;
  const float ag = fabsf(g), au = fabsf(u);
  const float t1 = __builtin_amdgcn_exp2f(-2.0f * kLog2e * inv_beta * ag);
  const float t2 = __builtin_amdgcn_exp2f(-2.0f * kLog2e * inv_lam * au);
  const float sg = __builtin_amdgcn_exp2f(-kLog2e * ag);
  const float num = (1.0f - t1) * (1.0f - t2) * (g >= 0.0f ? 1.0f : sg);
  const float den = (1.0f + t1) * (1.0f + t2) * (1.0f + sg);
  const float mag = beta * lam * num * __builtin_amdgcn_rcpf(den);
  return ((g < 0.0f) != (u < 0.0f)) ? -mag : mag;
}


// ---------------------------------------------------------------------------------------
// NW waves per workgroup, WRG 16-row MFMA groups per wave, up to BN tokens per tile.
template <int MODE, int NW, int WRG, int BN>
struct GemmCfg {
  static constexpr int kThreads = NW * 64;
  static constexpr int kNcb = BN / 16;                 // 16-token MFMA column blocks
  static constexpr int kWgRows = NW * WRG * 16;        // weight rows per workgroup
};

// Everything a workgroup needs once its tile is known.  The expert's prepared codes and
// scales are addressed through buffer resources: a load's offset is a wave-uniform part
// (row group, chunk) in a scalar register plus a fixed per-lane part.
struct TileCtx {
  TileDesc td;
  int e, tid, lane, w, g;
  int nchunks, groups, G0;
  __amdgpu_buffer_rsrc_t wcodes, wscales;   // this expert's prepared codes / scales
  uint32_t lane_code_off, lane_scale_off;
};

template <int WRG, int POLICY>
__device__ __forceinline__ void load_weights(const TileCtx& t, int c, uint4 (&wc)[WRG],
                                             uint32_t (&ws)[WRG]) {
#pragma unroll
  for (int r = 0; r < WRG; ++r) {
    const uint32_t chunk = static_cast<uint32_t>(c * t.groups + t.G0 + r);
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(t.wcodes, t.lane_code_off,
                                                          chunk * 1024u, POLICY);
    wc[r] = uint4{v[0], v[1], v[2], v[3]};
    ws[r] = __builtin_amdgcn_raw_buffer_load_b32(t.wscales, t.lane_scale_off, chunk * 128u, POLICY);
  }
}

// ---------------------------------------------------------------------------------------
// Token-tile staging: how a 128-column chunk of the tile's token rows gets from memory
// into an LDS buffer of f16 MFMA operands.  `load` fills registers (issued two chunks
// ahead), `store` writes them into a buffer, `frag` addresses a lane's operand: the 8
// values k = 32s + 8(lane/16) .. +7 of tile row 16cb + lane%16.  Only the first ROWS
// rows (a multiple of 16) are staged.

// FC1: the rows of x_dec (x's NVFP4 values in f16, written by the quantizer), moved as
// 16-byte pieces.  One load instruction of a wave covers 4 rows x 256 bytes (lane:
// row r0 + lane/16, piece lane%16), so each row is read as one contiguous 256-byte
// segment.  LDS rows are 128 f16 without padding; piece j of row r sits in slot
// j ^ (r % 16), so the 16 rows of an operand read hit 16 different slots.
template <int NW, int BN>
struct RowStage {
  static constexpr int kTileRows = BN;
  static constexpr int kPieces = BN / (4 * NW);        // 16-byte pieces per thread
  static constexpr int kLdsRow = kChunk;
  static_assert(BN % (4 * NW) == 0, "row staging split");
  struct Regs { u32x4 v[kPieces]; };
  const uint16_t* src;
  int32_t off[kPieces];                                // element offset in chunk 0
  int lds0, w;

  __device__ __forceinline__ void init(const LayerArgs& a, const int64_t* s_row, int wave,
                                       int lane) {
    src = a.x_dec;
    w = wave;
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int r = (i * NW + wave) * 4 + (lane >> 4);
      const int j = (lane & 15) ^ (r & 15);
      off[i] = static_cast<int32_t>(s_row[r] * a.H) + 8 * j;
    }
    lds0 = (wave * 4 + (lane >> 4)) * kLdsRow + 8 * (lane & 15);
  }
  // piece i of this wave lies in the first ROWS rows (decided at compile time unless the
  // staged rows end inside piece i's group of NW waves)
  template <int ROWS>
  __device__ __forceinline__ bool covers(int i) const {
    return (i + 1) * NW * 4 <= ROWS || (i * NW * 4 < ROWS && (i * NW + w) * 4 < ROWS);
  }
  template <int ROWS>
  __device__ __forceinline__ void load(int c, Regs& R) const {
#pragma unroll
    for (int i = 0; i < kPieces; ++i)
      if (covers<ROWS>(i))
        R.v[i] = *reinterpret_cast<const u32x4*>(src + off[i] + c * kChunk);
  }
  template <int ROWS>
  __device__ __forceinline__ void store(_Float16* buf, const Regs& R) const {
#pragma unroll
    for (int i = 0; i < kPieces; ++i)
      if (covers<ROWS>(i))
        *reinterpret_cast<u32x4*>(buf + lds0 + i * NW * 4 * kLdsRow) = R.v[i];
  }
  static __device__ __forceinline__ const _Float16* frag(const _Float16* buf, int cb, int s,
                                                         int lane) {
    return buf + (cb * 16 + (lane & 15)) * kLdsRow + 8 * ((4 * s + (lane >> 4)) ^ (lane & 15));
  }
};

// NVFP4 codes (x for FC1, the requantized SiTU rows for FC2), decoded to f16 on the way
// into LDS.  Each row's 64 code bytes per chunk are split over NW*64/BN threads (kNdw
// dwords each, read through buffer resources); columns past the row's real length (FC2's
// padded I) read as zero codes with a zero scale.  LDS rows are padded by 16 bytes.
template <int MODE, int NW, int BN>
struct CodeStage {
  static constexpr int kTileRows = BN;
  static constexpr int kThreadsPerRow = NW * 64 / BN;
  static constexpr int kNdw = 16 / kThreadsPerRow;     // code dwords (of 16 per row)
  static constexpr int kLdsRow = kChunk + 8;
  static_assert((NW * 64) % BN == 0 && 16 % kThreadsPerRow == 0, "code staging split");
  static_assert(kNdw == 2 || kNdw == 4 || kNdw == 8, "code staging width");
  struct Regs { uint32_t w[kNdw]; uint32_t sc; };
  __amdgpu_buffer_rsrc_t codes, scales;
  uint32_t code_off, scale_off;                        // this thread's bytes in chunk 0
  int trow, part_byte, valid_code_bytes;

  __device__ __forceinline__ void init(const LayerArgs& a, const int64_t* s_row, int wave,
                                       int lane) {
    const int tid = wave * 64 + lane;
    trow = tid / kThreadsPerRow;
    part_byte = (tid % kThreadsPerRow) * kNdw * 4;
    const int K = MODE == 0 ? a.H : a.I;
    const int64_t nrows = MODE == 0 ? a.T : static_cast<int64_t>(a.T) * a.k;
    codes = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(MODE == 0 ? a.x_codes : a.a_codes), 0,
        static_cast<int>(nrows * (K / 2)), kBufferFlags);
    scales = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(MODE == 0 ? a.x_scales : a.a_scales), 0,
        static_cast<int>(nrows * (K / 16)), kBufferFlags);
    code_off = static_cast<uint32_t>(s_row[trow] * (K / 2) + part_byte);
    scale_off = static_cast<uint32_t>(s_row[trow] * (K / 16) + part_byte / 8);
    valid_code_bytes = K / 2;
  }
  template <int ROWS>
  __device__ __forceinline__ void load(int c, Regs& R) const {
    if (trow >= ROWS) return;
    if (c * 64 + part_byte < valid_code_bytes) {
      const uint32_t co = code_off + 64u * c, so = scale_off + 8u * c;
#pragma unroll
      for (int i = 0; i < kNdw; i += (kNdw >= 4 ? 4 : 2)) {
        if constexpr (kNdw >= 4) {
          const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(codes, co + 4 * i, 0, 0);
          R.w[i] = v[0]; R.w[i + 1] = v[1]; R.w[i + 2] = v[2]; R.w[i + 3] = v[3];
        } else {
          const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(codes, co + 4 * i, 0, 0);
          R.w[i] = v[0]; R.w[i + 1] = v[1];
        }
      }
      // kNdw dwords = kNdw/2 blocks = kNdw/2 scale bytes
      if constexpr (kNdw == 8) R.sc = __builtin_amdgcn_raw_buffer_load_b32(scales, so, 0, 0);
      else if constexpr (kNdw == 4) R.sc = __builtin_amdgcn_raw_buffer_load_b16(scales, so, 0, 0);
      else R.sc = __builtin_amdgcn_raw_buffer_load_b8(scales, so, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < kNdw; ++i) R.w[i] = 0;
      R.sc = 0;
    }
  }
  template <int ROWS>
  __device__ __forceinline__ void store(_Float16* buf, const Regs& R) const {
    if (trow >= ROWS) return;
    _Float16* dst = buf + trow * kLdsRow + part_byte * 2;
#pragma unroll
    for (int i = 0; i < kNdw; ++i) {
      const f16x8 v = decode8(R.w[i], scale_f16x2_of(R.sc, i >> 1));
      *reinterpret_cast<f16x8*>(dst + 8 * i) = v;
    }
  }
  static __device__ __forceinline__ const _Float16* frag(const _Float16* buf, int cb, int s,
                                                         int lane) {
    return buf + (cb * 16 + (lane & 15)) * kLdsRow + 32 * s + 8 * (lane >> 4);
  }
};

// Staging of a variant: f16 rows (ROWS true, FC1 only) or NVFP4 codes.
template <int MODE, int NW, int BN, bool ROWS>
using StageOf = typename std::conditional<ROWS, RowStage<NW, BN>, CodeStage<MODE, NW, BN>>::type;

// One 128-column chunk c.  Weights run two chunks ahead in registers (on entry `wc/ws`
// hold chunk c's raw weights), tokens one chunk ahead through `tr`:
//   1. decode chunk c's weight fragments (frees wc/ws),
//   2. issue the loads of chunk c+2's weights (into wc/ws) and chunk c+1's tokens (tr),
//   3. wait for the LDS buffer of chunk c,
//   4. run the MFMAs,
//   5. store chunk c+1's tokens into the other LDS buffer.
//
// With WRG == 4 the weight fragments are decoded one 32-column K-step at a time and
// software-pipelined: step s+1's fragments are decoded while step s's MFMAs run.  Chunk
// c+2's weight loads are issued in step 3, after the last decode of chunk c.  The LDS
// operand of each 16-token block is read two blocks ahead, across K-steps within the
// chunk, and each fragment's block scale comes from one packed FP8 -> f16 conversion.
template <int WRG, int NCBA, int DEPTH, class Stage>
__device__ __forceinline__ void chunk_step(const TileCtx& t, const Stage& st, int c,
                                           uint4 (&wc)[WRG], uint32_t (&ws)[WRG],
                                           typename Stage::Regs& tr, const _Float16* tb_cur,
                                           _Float16* tb_next, f32x4 (&acc)[WRG][NCBA]) {
  constexpr bool kPerStep = WRG >= 4;
  auto decode_from = [&](const uint4 (&rc)[WRG], const uint32_t (&rs)[WRG], int s,
                         f16x8 (&dst)[WRG]) {
#pragma unroll
    for (int r = 0; r < WRG; ++r) {
      const uint32_t cw = s == 0 ? rc[r].x : s == 1 ? rc[r].y : s == 2 ? rc[r].z : rc[r].w;
      dst[r] = decode8(cw, scale_f16x2_of(rs[r], s));
    }
  };
  if constexpr (kPerStep) {
    const bool more = c + 1 < t.nchunks;
    st.template load<16 * NCBA>(min(c + 1, t.nchunks - 1), tr);
    __syncthreads();                                    // LDS buffer of chunk c complete
    f16x8 wf0[WRG], wf1[WRG];
    decode_from(wc, ws, 0, wf0);
    // The token operands of the chunk's 4*NCBA (K-step, block) items, in order, are read
    // two items ahead of their MFMAs.
    constexpr int kItems = 4 * NCBA;
    auto frag_of = [&](int i) {
      return *reinterpret_cast<const f16x8*>(Stage::frag(tb_cur, i % NCBA, i / NCBA, t.lane));
    };
    f16x8 xf = frag_of(0);
    f16x8 x1 = kItems > 1 ? frag_of(1) : xf;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      f16x8 (&cur)[WRG] = (s & 1) ? wf1 : wf0;
      f16x8 (&nxt)[WRG] = (s & 1) ? wf0 : wf1;
      if (s < 3) decode_from(wc, ws, s + 1, nxt);
      else load_weights<WRG, weight_load_policy(Stage::kTileRows)>(t, min(c + DEPTH, t.nchunks - 1), wc, ws);
#pragma unroll
      for (int cb = 0; cb < NCBA; ++cb) {
        const int i = s * NCBA + cb;
        const f16x8 x2 = i + 2 < kItems ? frag_of(i + 2) : x1;
#pragma unroll
        for (int r = 0; r < WRG; ++r) acc[r][cb] = mfma16x16x32(cur[r], xf, acc[r][cb]);
        xf = x1;
        x1 = x2;
      }
#pragma unroll
      for (int cb = 0; cb < NCBA; ++cb) {
        if (s * NCBA + cb + 2 < kItems) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
        for (int r = 0; r < WRG; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);    // VALU (next decode)
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (more) st.template store<16 * NCBA>(tb_next, tr);
    return;
  }
  f16x8 wf[4][WRG];
#pragma unroll
  for (int s = 0; s < 4; ++s) decode_from(wc, ws, s, wf[s]);
  // Token loads first, so the wait before their LDS store (end of this step) leaves the
  // younger weight loads in flight.  Both are issued unconditionally (chunk index clamped,
  // the surplus loads are never used): with no branch around them the compiler's wait
  // counts stay exact instead of draining every outstanding load.
  const bool more = c + 1 < t.nchunks;
  st.template load<16 * NCBA>(min(c + 1, t.nchunks - 1), tr);
  load_weights<WRG, weight_load_policy(Stage::kTileRows)>(t, min(c + DEPTH, t.nchunks - 1), wc, ws);
  __syncthreads();                                      // LDS buffer of chunk c complete
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int cb = 0; cb < NCBA; ++cb) {
      const f16x8 xf = *reinterpret_cast<const f16x8*>(Stage::frag(tb_cur, cb, s, t.lane));
#pragma unroll
      for (int r = 0; r < WRG; ++r) acc[r][cb] = mfma16x16x32(wf[s][r], xf, acc[r][cb]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (more) st.template store<16 * NCBA>(tb_next, tr);
}

template <int MODE, int NW, int WRG, int BN, bool ROWS, int NCBA>
__device__ __forceinline__ void tile_body(const LayerArgs& a, const TileCtx& t,
                                          const StageOf<MODE, NW, BN, ROWS>& st,
                                          _Float16 (*s_tok)[BN * StageOf<MODE, NW, BN, ROWS>::kLdsRow],
                                          float* s_enc) {
  using Stage = StageOf<MODE, NW, BN, ROWS>;
  f32x4 acc[WRG][NCBA];
#pragma unroll
  for (int i = 0; i < WRG; ++i)
#pragma unroll
    for (int j = 0; j < NCBA; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // DEPTH register sets of raw weights: set i holds chunk c+i on entry to chunk c's step
  // (deeper prefetch measured no faster: the small tiles lose occupancy, the big ones
  // have no registers left)
  constexpr int DEPTH = 2;
  uint4 wc[DEPTH][WRG];
  uint32_t ws[DEPTH][WRG];
  typename Stage::Regs tr;
#pragma unroll
  for (int i = 0; i < DEPTH; ++i) load_weights<WRG, weight_load_policy(BN)>(t, min(i, t.nchunks - 1), wc[i], ws[i]);
  st.template load<16 * NCBA>(0, tr);
  st.template store<16 * NCBA>(s_tok[0], tr);
  // DEPTH chunks per trip so register sets and LDS buffers are named statically; the
  // remaining chunks are peeled after the loop
  int c = 0;
  for (; c + DEPTH <= t.nchunks; c += DEPTH) {
#pragma unroll
    for (int i = 0; i < DEPTH; ++i)
      chunk_step<WRG, NCBA, DEPTH>(t, st, c + i, wc[i], ws[i], tr, s_tok[i & 1],
                                   s_tok[(i + 1) & 1], acc);
  }
#pragma unroll
  for (int i = 0; i + 1 < DEPTH; ++i)
    if (c + i < t.nchunks)
      chunk_step<WRG, NCBA, DEPTH>(t, st, c + i, wc[i], ws[i], tr, s_tok[i & 1],
                                   s_tok[(i + 1) & 1], acc);

  const TileDesc td = t.td;
  const int e = t.e, lane = t.lane, g = t.g, G0 = t.G0;
  if constexpr (MODE == 0) {
    // Lane holds rows 4g..4g+3 of each group = (gate i, up i, gate i+1, up i+1),
    // i = 8G + 2g.  Groups (2p, 2p+1) of the wave form NVFP4 group G0/2 + p.
    const float al = a.alpha1[e];
    const float qa = a.qa[e];
    // the encode factor of every scale byte, once per tile (s_enc is read only below)
    if (t.tid < 128) s_enc[t.tid] = nvfp4_encode_factor(t.tid, qa);
    __syncthreads();
    const float beta = a.beta ? a.beta[e] : 4.0f;
    const float lam = a.lam ? a.lam[e] : 25.0f;
    const float ib = 1.0f / beta, il = 1.0f / lam;
    float wave_amax = 0.0f;
#pragma unroll
    for (int cb = 0; cb < NCBA; ++cb) {
      const int n = cb * 16 + (lane & 15);
      const bool valid = n < td.nrows;
      const int64_t row = td.row_start + n;
#pragma unroll
      for (int p = 0; p < WRG / 2; ++p) {
        float av[4];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const f32x4 h = acc[2 * p + q][cb];
          av[2 * q] = situ(h[0] * al, h[1] * al, beta, ib, lam, il);
          av[2 * q + 1] = situ(h[2] * al, h[3] * al, beta, ib, lam, il);
        }
        float m = fmaxf(fmaxf(fabsf(av[0]), fabsf(av[1])), fmaxf(fabsf(av[2]), fabsf(av[3])));
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        if (valid) wave_amax = fmaxf(wave_amax, m);
        const uint32_t sb = nvfp4_scale_byte(m, qa);
        const float enc = s_enc[sb];
        const uint32_t w2 =
            e2m1_pack2<1>(e2m1_pack2<0>(0u, av[0] * enc, av[1] * enc), av[2] * enc, av[3] * enc);
        const uint32_t b0 = w2 & 0xFFu, b1 = (w2 >> 8) & 0xFFu;
        const int blk = (G0 >> 1) + p;
        if (valid) {
          uint8_t* ac = a.a_codes + row * (a.I / 2) + 8 * blk;
          ac[g] = static_cast<uint8_t>(b0);
          ac[4 + g] = static_cast<uint8_t>(b1);
          if (g == 0) a.a_scales[row * (a.I / 16) + blk] = static_cast<uint8_t>(sb);
        }
      }
    }
    for (int off = 32; off > 0; off >>= 1) wave_amax = fmaxf(wave_amax, __shfl_xor(wave_amax, off));
    if (lane == 0 && wave_amax > 0.0f)
      atomicMax(reinterpret_cast<unsigned int*>(a.a_amax + e), __float_as_uint(wave_amax));
  } else {
    // the K loop's token buffers are free once every wave has passed its last chunk; each
    // wave then stages its output blocks in its own part of them
    static_assert(2 * BN * Stage::kLdsRow >= NW * 16 * out_lds_stride<WRG>(),
                  "output staging space");
    __syncthreads();
    uint16_t* lds = reinterpret_cast<uint16_t*>(&s_tok[0][0]) + t.w * 16 * out_lds_stride<WRG>();
    const OutScale osc = out_scale(a.alpha2[e], a.I);
#pragma unroll
    for (int cb = 0; cb < NCBA; ++cb) {
      // stored at the row's flat id t*k + j (the finalization reads a token's rows as
      // one contiguous run)
      const int n = min(cb * 16 + (lane & 15), td.nrows - 1);
      const int32_t flat = a.sorted_row_idx[td.row_start + n];
      f32x4 blk[WRG];
#pragma unroll
      for (int r = 0; r < WRG; ++r) blk[r] = acc[r][cb];
      store_out_block<WRG>(blk, osc, lds, lane, flat, td.nrows - cb * 16, a.o_rows, a.o_exp,
                           a.H, 16 * G0);
    }
  }
}

// Consecutive logical workgroups kept on one XCD.  FC1 with code-staged token tiles (many
// routed rows) keeps a whole group of kTileGroup token tiles with all its n_wt slabs on one
// XCD, so that the group's token rows, reread for every slab, and each slab's weights,
// reread for every tile, are both fetched into one L2; elsewhere kXcdRun.
template <int MODE, bool ROWS>
__host__ __device__ constexpr int xcd_run(int n_wt) {
  return MODE == 0 && !ROWS ? kTileGroup * n_wt : kXcdRun;
}

// The LDS of one workgroup of a variant: the double-buffered token tile, the tile's
// token rows and (FC1's requantization) the encode factor qa/s of every E4M3 scale byte s
// of the tile's expert, divided once per tile instead of once per 16-value block.
template <int MODE, int NW, int BN, bool ROWS>
struct GemmLds {
  _Float16 tok[2][BN * StageOf<MODE, NW, BN, ROWS>::kLdsRow];
  int64_t row[BN];
  float enc[128];
};

// Workgroup b of a variant's grid (b counts from the variant's first workgroup; the grid
// starts at a multiple of the XCD count): token tile and weight slab from b, then the tile
// body.
template <int MODE, int NW, int WRG, int BN, bool ROWS>
__device__ __forceinline__ void gemm_workgroup(const LayerArgs& a, int big, int b,
                                               GemmLds<MODE, NW, BN, ROWS>& L) {
  using C = GemmCfg<MODE, NW, WRG, BN>;
  using Stage = StageOf<MODE, NW, BN, ROWS>;
  auto& s_tok = L.tok;
  int64_t* s_row = L.row;
  float* s_enc = L.enc;
  const TileDesc* tiles = big ? a.tiles_big : a.tiles_small;
  const int ntiles = a.num_tiles[big];
  const int rows_total = MODE == 0 ? 2 * a.I : a.H;
  const int n_wt = rows_total / C::kWgRows;
  int tt, wt;
  map_workgroup(b, n_wt, a.xcds, &tt, &wt, xcd_run<MODE, ROWS>(n_wt));
  if (tt >= ntiles) return;
  TileCtx t;
  t.td = tiles[tt];
  t.e = t.td.expert;
  t.tid = threadIdx.x; t.lane = t.tid & 63; t.w = t.tid >> 6; t.g = t.lane >> 4;
  if (t.tid < BN) {
    const int r = t.td.row_start + min(t.tid, t.td.nrows - 1);
    s_row[t.tid] = MODE == 0 ? static_cast<int64_t>(a.sorted_row_idx[r] / a.k) : r;
  }
  __syncthreads();
  const int K = MODE == 0 ? a.H : a.Ip;
  t.nchunks = K / kChunk;
  const int RG = rows_total / 16;
  t.G0 = wt * (C::kWgRows / 16) + __builtin_amdgcn_readfirstlane(t.w) * WRG;
  {
    // this expert's chunks (prepared_chunk): (chunk c, row group G) -> 64 lanes x 16 code
    // bytes at (c*groups + G) * 1024 and 128 scale bytes at (c*groups + G) * 128
    t.groups = RG;
    const int64_t expert_chunks = static_cast<int64_t>(RG) * t.nchunks;
    const uint8_t* wc = (MODE == 0 ? a.w13_codes : a.w2_codes) + t.e * expert_chunks * 1024;
    const uint8_t* wsc = (MODE == 0 ? a.w13_scales : a.w2_scales) + t.e * expert_chunks * 128;
    t.wcodes = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(wc), 0,
                                                 static_cast<int>(expert_chunks * 1024), kBufferFlags);
    t.wscales = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(wsc), 0,
                                                  static_cast<int>(expert_chunks * 128), kBufferFlags);
    t.lane_code_off = 16u * t.lane;
    t.lane_scale_off = 4u * static_cast<uint32_t>(prepared_scale_index(0, t.lane));
  }
  Stage st;
  st.init(a, s_row, t.w, t.lane);

  // one instantiation per number of active 16-token column blocks, so the MFMA loops
  // have compile-time trip counts (uniform branch per workgroup)
  const int ncb = (t.td.nrows + 15) / 16;
  if constexpr (BN == 32) {
    if (ncb == 1) tile_body<MODE, NW, WRG, BN, ROWS, 1>(a, t, st, s_tok, s_enc);
    else tile_body<MODE, NW, WRG, BN, ROWS, 2>(a, t, st, s_tok, s_enc);
  } else {
    switch (ncb) {
      case 1: tile_body<MODE, NW, WRG, BN, ROWS, 1>(a, t, st, s_tok, s_enc); break;
      case 2: tile_body<MODE, NW, WRG, BN, ROWS, 2>(a, t, st, s_tok, s_enc); break;
      case 3: tile_body<MODE, NW, WRG, BN, ROWS, 3>(a, t, st, s_tok, s_enc); break;
      case 4: tile_body<MODE, NW, WRG, BN, ROWS, 4>(a, t, st, s_tok, s_enc); break;
      case 5: tile_body<MODE, NW, WRG, BN, ROWS, 5>(a, t, st, s_tok, s_enc); break;
      case 6: tile_body<MODE, NW, WRG, BN, ROWS, 6>(a, t, st, s_tok, s_enc); break;
      default: tile_body<MODE, NW, WRG, BN, ROWS, 7>(a, t, st, s_tok, s_enc); break;   // kBigTileRows
    }
  }
}


template <int MODE, int NW, int WRG, int BN, int WPE, bool ROWS>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
void grouped_gemm_kernel(LayerArgs a, int big) {
  __shared__ GemmLds<MODE, NW, BN, ROWS> lds;
  gemm_workgroup<MODE, NW, WRG, BN, ROWS>(a, big, blockIdx.x, lds);
}

// Both tile lists in one launch: the big tiles' workgroups first (the longest, so they
// start first), then the small tiles' in the rest of the grid.  The two kinds run side by
// side: the big tiles of a skewed batch's hot experts are few, long and MFMA-heavy, the
// small tiles many and bound by the weight stream.
template <int MODE, int NW, int WRG_B, int BN_B, int WRG_S, int BN_S, int WPE, bool ROWS>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
void grouped_gemm_pair_kernel(LayerArgs a, int grid_big) {
  using LB = GemmLds<MODE, NW, BN_B, ROWS>;
  using LS = GemmLds<MODE, NW, BN_S, ROWS>;
  __shared__ __attribute__((aligned(16))) char lds[sizeof(LB) > sizeof(LS) ? sizeof(LB) : sizeof(LS)];
  if (static_cast<int>(blockIdx.x) < grid_big)
    gemm_workgroup<MODE, NW, WRG_B, BN_B, ROWS>(a, 1, blockIdx.x, *reinterpret_cast<LB*>(lds));
  else
    gemm_workgroup<MODE, NW, WRG_S, BN_S, ROWS>(a, 0, blockIdx.x - grid_big,
                                                *reinterpret_cast<LS*>(lds));
}

// out[t, 8v..8v+7] = BF16(sum_j w[t, j] * o[t*k + j, 8v..8v+7]), j in order, fp32 fused
// multiply-add; rows whose id was dropped (gather-map entry < 0) are skipped.  FC2 stored
// the rows in flat id order, so a token's k rows are one contiguous run; a stored value is
// o * 2^s with s the exponent of its row (its expert's), so it enters the sum with the
// weight w * 2^-s (exact).  A workgroup covers up to 8*kFinThreads columns of one token; each
// thread owns 8 columns and issues the 16-byte loads of NB rows at a time before it
// accumulates them.  The row loads do not wait for the gather map: every row t*k + j lies
// in the FC2 output, and a dropped row's (unwritten) values are loaded but not used, so
// the map, weight, exponent and row loads of a batch are in flight together.
constexpr int kFinThreads = 512;

// VEC: k is a multiple of NB, so a batch's exponents are one NB-byte load; else one byte
// load per row (index clamped: every load is unconditional).
template <int NB, bool VEC>
__global__ __launch_bounds__(kFinThreads) void finalize_kernel(LayerArgs a, int col_blocks) {
  const int64_t t = blockIdx.x / col_blocks;
  const int v = (blockIdx.x % col_blocks) * blockDim.x + threadIdx.x;
  if (v >= a.H / 8) return;
  const int32_t* __restrict__ pos_t = a.expanded_row_idx + t * a.k;
  const uint16_t* __restrict__ w_t = a.route_weights + t * a.k;
  const int8_t* __restrict__ exp_t = a.o_exp + t * a.k;     // the token's k row exponents
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < a.k; j0 += NB) {
    u32x4 d[NB];
    int32_t sx[NB];
    bool ok[NB];
    uint32_t e4[NB / 4 > 0 ? NB / 4 : 1];
    if constexpr (VEC && NB == 16) {
      const uint4 q = *reinterpret_cast<const uint4*>(exp_t + j0);
      e4[0] = q.x; e4[1] = q.y; e4[2] = q.z; e4[3] = q.w;
    } else if constexpr (VEC && NB == 8) {
      const uint2 q = *reinterpret_cast<const uint2*>(exp_t + j0);
      e4[0] = q.x; e4[1] = q.y;
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int j = j0 + u, jc = min(j, a.k - 1);
      ok[u] = j < a.k && pos_t[jc] >= 0;        // < 0: dropped (expert id out of range)
      // read once, never again: nontemporal, so the rows do not displace cached data
      d[u] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(a.o_rows + (t * a.k + jc) * a.H) + v);
      if constexpr (VEC) sx[u] = static_cast<int8_t>((e4[u / 4] >> (8 * (u & 3))) & 0xFFu);
      else sx[u] = exp_t[jc];
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      if (!ok[u]) continue;
      const float wt = bf16_to_f32(w_t[min(j0 + u, a.k - 1)]) *
                       __uint_as_float(static_cast<uint32_t>(127 - sx[u]) << 23);
      const uint32_t dw[4] = {d[u][0], d[u][1], d[u][2], d[u][3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x2 o = __builtin_convertvector(__builtin_bit_cast(f16x2, dw[i]), f32x2);
        acc[2 * i] = fmaf(wt, o[0], acc[2 * i]);
        acc[2 * i + 1] = fmaf(wt, o[1], acc[2 * i + 1]);
      }
    }
  }
  uint4 o;
  o.x = pack_bf16x2(acc[0], acc[1]);
  o.y = pack_bf16x2(acc[2], acc[3]);
  o.z = pack_bf16x2(acc[4], acc[5]);
  o.w = pack_bf16x2(acc[6], acc[7]);
  reinterpret_cast<uint4*>(a.out + t * a.H)[v] = o;
}


// Variants: small tiles (up to 32 tokens) run 4 waves x 4 groups (256-row slabs) in FC1
// and 4 waves x 2 groups (128-row slabs) in FC2 or when the rows do not divide, and stage
// FC1's tokens as f16 rows.  Big tiles (up to kBigRows tokens) run 4 waves x 2
// groups, FC1 with f16 rows; with at least two big tiles per CU of routed rows
// (many_rows) FC1's big tiles run 4 waves x 4 groups instead (half the LDS operand reads per
// MFMA; the tokens are staged as codes, a quarter of the f16 rows' bytes: each token row is
// fetched once per slab, so f16 rows would double the kernel's memory traffic).
// A slab that does not divide the rows falls back to 128-row slabs.
constexpr int kBigNW = 4, kBigWRG = 2, kBigWPE = 2;
constexpr int kFc1WideWRG = 4, kFc1WideWPE = 2;
// FC1 small tiles: 4 row groups per wave (256-row slabs) beside big tiles; in batches of
// small tiles only, 6 (384-row slabs: each expert's 2I = 768 rows in two workgroups
// instead of three, so each streams a longer run of weights; T=64 FC1 -5%).
constexpr int kFc1SmallWRG = 4, kFc1SmallOnlyWRG = 6;

template <int MODE, int NW, int WRG, int BN, bool ROWS>
static int64_t variant_grid(const LayerArgs& a, int64_t max_tiles) {
  using C = GemmCfg<MODE, NW, WRG, BN>;
  const int rows_total = MODE == 0 ? 2 * a.I : a.H;
  const int n_wt = rows_total / C::kWgRows;
  return round_up(round_up(max_tiles, kTileGroup) * n_wt,
                  static_cast<int64_t>(a.xcds) * xcd_run<MODE, ROWS>(n_wt));
}

template <int MODE, int NW, int WRG, int BN, int WPE, bool ROWS>
static void launch_variant(const LayerArgs& a, int64_t max_tiles, int big, hipStream_t stream) {
  using C = GemmCfg<MODE, NW, WRG, BN>;
  const int64_t grid = variant_grid<MODE, NW, WRG, BN, ROWS>(a, max_tiles);
  if (grid > 0)
    grouped_gemm_kernel<MODE, NW, WRG, BN, WPE, ROWS>
        <<<dim3(static_cast<unsigned>(grid)), dim3(C::kThreads), 0, stream>>>(a, big);
}

// Both of FC1's tile lists in one launch (grouped_gemm_pair_kernel), 4-wave workgroups.
template <int WRG_B, int WRG_S, int WPE, bool ROWS>
static void launch_fc1_pair(const LayerArgs& a, hipStream_t stream) {
  const int64_t gb = variant_grid<0, 4, WRG_B, kBigRows, ROWS>(a, a.max_big);
  const int64_t gs = variant_grid<0, 4, WRG_S, kSmallRows, ROWS>(a, a.max_small);
  if (gb + gs > 0)
    grouped_gemm_pair_kernel<0, 4, WRG_B, kBigRows, WRG_S, kSmallRows, WPE, ROWS>
        <<<dim3(static_cast<unsigned>(gb + gs)), dim3(256), 0, stream>>>(a, static_cast<int>(gb));
}

template <int MODE>
static hipError_t launch_gemm(const LayerArgs& a, hipStream_t stream) {
  constexpr bool kRows = MODE == 0;
  const int rows_total = MODE == 0 ? 2 * a.I : a.H;
  const bool many = many_rows(static_cast<int64_t>(a.T) * a.k, a.cus);
  const bool small_wide =
      MODE == 0 && rows_total % GemmCfg<MODE, 4, kFc1SmallWRG, kSmallRows>::kWgRows == 0;
  if (kRows && many) {
    if constexpr (MODE == 0) {
      // Both lists in one launch: a batch this large has few small tiles (none when the
      // routing is even), and their workgroups then finish the big tiles' grid instead of
      // filling a launch of their own.
      if (small_wide && rows_total % GemmCfg<MODE, kBigNW, kFc1WideWRG, kBigRows>::kWgRows == 0) {
        static_assert(kBigNW == 4, "one workgroup size for both tile kinds");
        launch_fc1_pair<kFc1WideWRG, kFc1SmallWRG, kFc1WideWPE, false>(a, stream);
        return hipGetLastError();
      }
    }
    // no f16 copy of x: the small tiles stage codes too
    if (small_wide) launch_variant<MODE, 4, kFc1SmallWRG, kSmallRows, 2, false>(a, a.max_small, 0, stream);
    else launch_variant<MODE, 4, 2, kSmallRows, 1, false>(a, a.max_small, 0, stream);
  } else if (small_wide) {
    if constexpr (MODE == 0) {
      // a batch with big tiles and f16 rows of x (the mid-size batches): both lists in one
      // launch
      const bool pair = static_cast<int64_t>(a.T) * a.k > kSmallOnlyRows &&
                        rows_total % GemmCfg<MODE, kBigNW, kBigWRG, kBigRows>::kWgRows == 0;
      if (pair) {
        launch_fc1_pair<kBigWRG, kFc1SmallWRG, kBigWPE, true>(a, stream);
        return hipGetLastError();
      }
    }
    if constexpr (MODE == 0) {
      if (static_cast<int64_t>(a.T) * a.k <= kSmallOnlyRows &&
          rows_total % GemmCfg<MODE, 4, kFc1SmallOnlyWRG, kSmallRows>::kWgRows == 0) {
        launch_variant<MODE, 4, kFc1SmallOnlyWRG, kSmallRows, 2, kRows>(a, a.max_small, 0, stream);
        return hipGetLastError();
      }
    }
    launch_variant<MODE, 4, kFc1SmallWRG, kSmallRows, 2, kRows>(a, a.max_small, 0, stream);
  } else {
    launch_variant<MODE, 4, 2, kSmallRows, 1, kRows>(a, a.max_small, 0, stream);
  }
  // batches of at most kSmallOnlyRows routed rows have small tiles only
  if (static_cast<int64_t>(a.T) * a.k <= kSmallOnlyRows) return hipGetLastError();
  // (with many rows there is no f16 copy of x: FC1's fallback slabs stage codes too)
  const bool big_slabs = rows_total % GemmCfg<MODE, kBigNW, kBigWRG, kBigRows>::kWgRows == 0;
  if (kRows && many) {
    if (big_slabs) launch_variant<MODE, kBigNW, kBigWRG, kBigRows, kBigWPE, false>(a, a.max_big, 1, stream);
    else launch_variant<MODE, 4, 2, kBigRows, 1, false>(a, a.max_big, 1, stream);
  } else if (big_slabs) {
    launch_variant<MODE, kBigNW, kBigWRG, kBigRows, kBigWPE, kRows>(a, a.max_big, 1, stream);
  } else {
    launch_variant<MODE, 4, 2, kBigRows, 1, kRows>(a, a.max_big, 1, stream);
  }
  return hipGetLastError();
}

// Fused FC1 + FC2 for batches with at most one routed row per compute unit (so at most
// that many small tiles, one per CU): a workgroup of kFusedNW waves takes one small tile
// and runs FC1 over all 2I rows of its expert in one sweep (WRG1 = 2I/(16*kFusedNW) row
// groups per wave, the same tile body as the FC1 kernels), then, once its intermediate
// codes are written, stages them as FC2's token tile and sweeps all H/(64*kFusedNW) FC2
// slabs of kFusedNW waves x 4 row groups over it (the FC2 tile body).  There is no launch
// boundary between FC1 and FC2, and each CU streams its expert's FC1 and FC2 weights back
// to back with every wave of the workgroup loading.
constexpr int kFusedNW = 8;

template <int WRG1, int NCH>
__global__ __launch_bounds__(kFusedNW * 64) void layer_small_fused_kernel(LayerArgs a) {
  using Stage = StageOf<0, kFusedNW, kSmallRows, true>;
  __shared__ _Float16 s_tok[2][kSmallRows * Stage::kLdsRow];
  __shared__ int64_t s_row[kSmallRows];
  __shared__ float s_enc[128];
  __shared__ _Float16 s_tok2[kSmallRows * kFc2LdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t s_out[kFusedNW * 16 * out_lds_stride<4>()];
  static_assert(WRG1 % 2 == 0, "gate/up row-group pairs per wave");

  const int tt = blockIdx.x;
  if (tt >= a.num_tiles[0]) return;
  TileCtx t;
  t.td = a.tiles_small[tt];
  t.e = t.td.expert;
  t.tid = threadIdx.x; t.lane = t.tid & 63; t.w = t.tid >> 6; t.g = t.lane >> 4;
  if (t.tid < kSmallRows) {
    const int r = t.td.row_start + min(t.tid, t.td.nrows - 1);
    s_row[t.tid] = static_cast<int64_t>(a.sorted_row_idx[r] / a.k);
  }
  __syncthreads();
  t.nchunks = a.H / kChunk;
  const int RG = 2 * a.I / 16;
  t.G0 = __builtin_amdgcn_readfirstlane(t.w) * WRG1;
  {
    t.groups = RG;
    const int64_t expert_chunks = static_cast<int64_t>(RG) * t.nchunks;
    const uint8_t* wc = a.w13_codes + t.e * expert_chunks * 1024;
    const uint8_t* wsc = a.w13_scales + t.e * expert_chunks * 128;
    t.wcodes = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(wc), 0,
                                                 static_cast<int>(expert_chunks * 1024), kBufferFlags);
    t.wscales = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(wsc), 0,
                                                  static_cast<int>(expert_chunks * 128), kBufferFlags);
    t.lane_code_off = 16u * t.lane;
    t.lane_scale_off = 4u * static_cast<uint32_t>(prepared_scale_index(0, t.lane));
  }
  Stage st;
  st.init(a, s_row, t.w, t.lane);
  const int ncb = (t.td.nrows + 15) / 16;
  if (ncb == 1) tile_body<0, kFusedNW, WRG1, kSmallRows, true, 1>(a, t, st, s_tok, s_enc);
  else tile_body<0, kFusedNW, WRG1, kSmallRows, true, 2>(a, t, st, s_tok, s_enc);
  __syncthreads();                        // the tile's intermediate codes are written
  fc2_stage_tile(a, t.td, ncb, s_tok2, t.tid, kFusedNW * 64);
  __syncthreads();
  const int n_slabs = a.H / (kFusedNW * 4 * 16);
  if (ncb == 1) fc2_tile<kFusedNW, 4, kSmallRows, 1, NCH>(a, t.td, 0, n_slabs, s_tok2, s_out);
  else fc2_tile<kFusedNW, 4, kSmallRows, 2, NCH>(a, t.td, 0, n_slabs, s_tok2, s_out);
}

bool layer_small_fused_fits(const LayerArgs& a) {
  const int64_t R = static_cast<int64_t>(a.T) * a.k;
  return R <= a.cus && R <= kSmallOnlyRows && a.I % 128 == 0 && a.I <= kFc2MaxIp &&
         a.I == a.Ip && a.H % (kFusedNW * 4 * 16) == 0;
}

hipError_t launch_layer_small_fused(const LayerArgs& a, hipStream_t stream) {
  const dim3 g(static_cast<unsigned>(a.max_small)), b(kFusedNW * 64);
  if (a.max_small == 0) return hipSuccess;
  switch (a.I / kChunk) {
    case 1: layer_small_fused_kernel<2, 1><<<g, b, 0, stream>>>(a); break;
    case 2: layer_small_fused_kernel<4, 2><<<g, b, 0, stream>>>(a); break;
    default: layer_small_fused_kernel<6, 3><<<g, b, 0, stream>>>(a); break;
  }
  return hipGetLastError();
}

hipError_t launch_fc1(const LayerArgs& a, hipStream_t stream) { return launch_gemm<0>(a, stream); }
hipError_t launch_fc2(const LayerArgs& a, hipStream_t stream) {
  if (!fc2_resident_fits(a)) return launch_gemm<1>(a, stream);
  launch_fc2_resident_small(a, stream);
  if (static_cast<int64_t>(a.T) * a.k <= kSmallOnlyRows) return hipGetLastError();
  // With fewer than about two big tiles per CU, each tile is spread over four workgroups
  // (two sub-tiles x two slab groups); with more, over two (sub-tiles, all slabs each).
  if (many_rows(static_cast<int64_t>(a.T) * a.k, a.cus)) launch_fc2_resident_big(a, stream);
  else if (a.H % 256 == 0) launch_fc2_resident_big_spread(a, stream);
  else if (a.H % GemmCfg<1, kBigNW, kBigWRG, kBigRows>::kWgRows == 0)
    launch_variant<1, kBigNW, kBigWRG, kBigRows, kBigWPE, false>(a, a.max_big, 1, stream);
  else
    launch_variant<1, 4, 2, kBigRows, 1, false>(a, a.max_big, 1, stream);
  return hipGetLastError();
}

hipError_t launch_finalize(const LayerArgs& a, hipStream_t stream) {
  // whole waves covering a token's H/8 vectors in as few workgroups as possible; a batch
  // of fewer than two tokens per CU splits each token's columns further (down to one wave
  // per workgroup), since one CU streams only a small share of the HBM bandwidth
  const int vecs = a.H / 8;
  const int min_blocks = (vecs + kFinThreads - 1) / kFinThreads;
  const int max_blocks = (vecs + 63) / 64;
  const int want = static_cast<int>((2 * static_cast<int64_t>(a.cus) + a.T - 1) / max(a.T, 1));
  const int col_blocks = max(min_blocks, min(want, max_blocks));
  const int per_block = (vecs + col_blocks - 1) / col_blocks;
  const int threads = (per_block + 63) / 64 * 64;
  const int64_t grid = static_cast<int64_t>(a.T) * col_blocks;
  const dim3 g(static_cast<unsigned>(grid)), b(threads);
  if (grid == 0) return hipSuccess;
  if (a.k % 16 == 0) finalize_kernel<16, true><<<g, b, 0, stream>>>(a, col_blocks);
  else if (a.k % 8 == 0) finalize_kernel<8, true><<<g, b, 0, stream>>>(a, col_blocks);
  else if (a.k > 8) finalize_kernel<16, false><<<g, b, 0, stream>>>(a, col_blocks);
  else finalize_kernel<8, false><<<g, b, 0, stream>>>(a, col_blocks);
  return hipGetLastError();
}

}  // namespace rmoe
