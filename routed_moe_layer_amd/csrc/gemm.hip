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
// per-expert amax statistic; the FC2 epilogue applies alpha2 and stores BF16 rows.
#include "common.h"
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
  static constexpr int kLdsRow = kChunk + 8;           // f16 per staged token row (+16 B pad)
  static constexpr int kThreadsPerRow = kThreads / BN; // token-decode threads per row
  static constexpr int kDwPerThread = 16 / kThreadsPerRow;   // code dwords (of 16 per row)
  static_assert(kThreads % BN == 0 && 16 % kThreadsPerRow == 0, "token decode split");
};

// Everything a workgroup needs once its tile is known.
struct TileCtx {
  TileDesc td;
  int e, tid, lane, w, g;
  int nchunks, G0;
  int64_t slot0;
  const uint4* wcodes;
  const uint32_t* wscales;
  const uint8_t* trow_codes;
  const uint8_t* trow_scales;
  int trow, tpart, valid_code_bytes;
};

template <int WRG>
__device__ __forceinline__ void load_weights(const TileCtx& t, int c, uint4 (&wc)[WRG],
                                             uint32_t (&ws)[WRG]) {
#pragma unroll
  for (int r = 0; r < WRG; ++r) {
    wc[r] = t.wcodes[((t.slot0 + r) * t.nchunks + c) * 64 + t.lane];
    ws[r] = t.wscales[prepared_scale_index(t.slot0 + r, t.nchunks, c, t.lane)];
  }
}

// Raw token codes and scale bytes of one chunk for one decoding thread.
template <int NDW>
struct TokRegs {
  uint32_t w[NDW];
  uint32_t sc;
};

// One 128-column chunk c.  Register pipelines run two chunks ahead: on entry `wc/ws` hold
// chunk c's raw weights and `tnext` chunk c+1's raw token codes; `tfree` is free.
//   1. decode chunk c's weight fragments (frees wc/ws),
//   2. issue the loads of chunk c+2 (weights into wc/ws, token codes into tfree),
//   3. wait for the LDS buffer of chunk c,
//   4. run the MFMAs,
//   5. decode chunk c+1's token codes into the other LDS buffer.
template <int WRG, int NCBA, int NDW, int LROW>
__device__ __forceinline__ void chunk_step(const TileCtx& t, int c, uint4 (&wc)[WRG],
                                           uint32_t (&ws)[WRG], TokRegs<NDW>& tfree,
                                           const TokRegs<NDW>& tnext, const _Float16* tb_cur,
                                           _Float16* tb_next, f32x4 (&acc)[WRG][NCBA]) {
  const bool tactive = t.trow < 16 * NCBA;
  f16x8 wf[4][WRG];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int r = 0; r < WRG; ++r) {
      const uint32_t cw = s == 0 ? wc[r].x : s == 1 ? wc[r].y : s == 2 ? wc[r].z : wc[r].w;
      wf[s][r] = decode8(cw, scale_f16x2((ws[r] >> (8 * s)) & 0xFFu));
    }
  if (c + 2 < t.nchunks) {
    load_weights<WRG>(t, c + 2, wc, ws);
    if (tactive)
      load_token_chunk<NDW>(t.trow_codes, t.trow_scales, c + 2, t.tpart, t.valid_code_bytes,
                            tfree.w, tfree.sc);
  }
  __syncthreads();                                      // LDS buffer of chunk c complete
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int cb = 0; cb < NCBA; ++cb) {
      const f16x8 xf = *reinterpret_cast<const f16x8*>(
          tb_cur + (cb * 16 + (t.lane & 15)) * LROW + 32 * s + 8 * t.g);
#pragma unroll
      for (int r = 0; r < WRG; ++r) acc[r][cb] = mfma16x16x32(wf[s][r], xf, acc[r][cb]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (c + 1 < t.nchunks && tactive)
    store_token_chunk<NDW>(tb_next + t.trow * LROW + t.tpart * NDW * 8, tnext.w, tnext.sc);
}

template <int MODE, int NW, int WRG, int BN, int NCBA>
__device__ __forceinline__ void tile_body(const LayerArgs& a, const TileCtx& t,
                                          _Float16 (*s_tok)[BN * GemmCfg<MODE, NW, WRG, BN>::kLdsRow]) {
  using C = GemmCfg<MODE, NW, WRG, BN>;
  constexpr int NDW = C::kDwPerThread;
  constexpr int LROW = C::kLdsRow;
  f32x4 acc[WRG][NCBA];
#pragma unroll
  for (int i = 0; i < WRG; ++i)
#pragma unroll
    for (int j = 0; j < NCBA; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 wcA[WRG], wcB[WRG];
  uint32_t wsA[WRG], wsB[WRG];
  TokRegs<NDW> tA, tB;
  const bool tactive = t.trow < 16 * NCBA;
  load_weights<WRG>(t, 0, wcA, wsA);
  if (t.nchunks > 1) load_weights<WRG>(t, 1, wcB, wsB);
  if (tactive) {
    load_token_chunk<NDW>(t.trow_codes, t.trow_scales, 0, t.tpart, t.valid_code_bytes, tA.w, tA.sc);
    store_token_chunk<NDW>(s_tok[0] + t.trow * LROW + t.tpart * NDW * 8, tA.w, tA.sc);
    if (t.nchunks > 1)
      load_token_chunk<NDW>(t.trow_codes, t.trow_scales, 1, t.tpart, t.valid_code_bytes, tB.w, tB.sc);
  }
  // two chunks per trip so register sets and LDS buffers are named statically; an odd
  // last chunk is peeled after the loop (no conditional MFMA block inside the loop)
  int c = 0;
  for (; c + 1 < t.nchunks; c += 2) {
    chunk_step<WRG, NCBA, NDW, LROW>(t, c, wcA, wsA, tA, tB, s_tok[0], s_tok[1], acc);
    chunk_step<WRG, NCBA, NDW, LROW>(t, c + 1, wcB, wsB, tB, tA, s_tok[1], s_tok[0], acc);
  }
  if (c < t.nchunks)
    chunk_step<WRG, NCBA, NDW, LROW>(t, c, wcA, wsA, tA, tB, s_tok[0], s_tok[1], acc);

  const TileDesc td = t.td;
  const int e = t.e, lane = t.lane, g = t.g, G0 = t.G0;
  if constexpr (MODE == 0) {
    // Lane holds rows 4g..4g+3 of each group = (gate i, up i, gate i+1, up i+1),
    // i = 8G + 2g.  Groups (2p, 2p+1) of the wave form NVFP4 group G0/2 + p.
    const float al = a.alpha1[e];
    const float qa = a.qa[e];
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
        float enc;
        const uint32_t sb = nvfp4_block_scale(m, qa, &enc);
        const uint32_t b0 = e2m1_encode(av[0] * enc) | (e2m1_encode(av[1] * enc) << 4);
        const uint32_t b1 = e2m1_encode(av[2] * enc) | (e2m1_encode(av[3] * enc) << 4);
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
    const float al = a.alpha2[e];
#pragma unroll
    for (int cb = 0; cb < NCBA; ++cb) {
      const int n = cb * 16 + (lane & 15);
      if (n >= td.nrows) continue;
      const int64_t row = td.row_start + n;
#pragma unroll
      for (int r = 0; r < WRG; ++r) {
        const f32x4 o = acc[r][cb];
        const int h0 = 16 * (G0 + r) + 4 * g;
        uint2 v;
        v.x = static_cast<uint32_t>(f32_to_bf16_rne(o[0] * al)) |
              (static_cast<uint32_t>(f32_to_bf16_rne(o[1] * al)) << 16);
        v.y = static_cast<uint32_t>(f32_to_bf16_rne(o[2] * al)) |
              (static_cast<uint32_t>(f32_to_bf16_rne(o[3] * al)) << 16);
        *reinterpret_cast<uint2*>(a.o_rows + row * a.H + h0) = v;
      }
    }
  }
}

template <int MODE, int NW, int WRG, int BN, int WPE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
void grouped_gemm_kernel(LayerArgs a, int big) {
  using C = GemmCfg<MODE, NW, WRG, BN>;
  __shared__ _Float16 s_tok[2][BN * C::kLdsRow];
  __shared__ int64_t s_row[BN];

  const TileDesc* tiles = big ? a.tiles_big : a.tiles_small;
  const int ntiles = a.num_tiles[big];
  const int rows_total = MODE == 0 ? 2 * a.I : a.H;
  const int n_wt = rows_total / C::kWgRows;
  int tt, wt;
  map_workgroup(blockIdx.x, n_wt, &tt, &wt);
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
  t.G0 = wt * (C::kWgRows / 16) + t.w * WRG;
  t.slot0 = static_cast<int64_t>(t.e) * RG + t.G0;
  t.wcodes = reinterpret_cast<const uint4*>(MODE == 0 ? a.w13_codes : a.w2_codes);
  t.wscales = reinterpret_cast<const uint32_t*>(MODE == 0 ? a.w13_scales : a.w2_scales);
  t.trow = t.tid / C::kThreadsPerRow;
  t.tpart = t.tid % C::kThreadsPerRow;
  const int64_t srow = s_row[t.trow];
  t.trow_codes = (MODE == 0 ? a.x_codes : a.a_codes) + srow * (MODE == 0 ? a.H / 2 : a.I / 2);
  t.trow_scales = (MODE == 0 ? a.x_scales : a.a_scales) + srow * (MODE == 0 ? a.H / 16 : a.I / 16);
  t.valid_code_bytes = MODE == 0 ? a.H / 2 : a.I / 2;

  // one instantiation per number of active 16-token column blocks, so the MFMA loops
  // have compile-time trip counts (uniform branch per workgroup)
  const int ncb = (t.td.nrows + 15) / 16;
  if constexpr (BN == 32) {
    if (ncb == 1) tile_body<MODE, NW, WRG, BN, 1>(a, t, s_tok);
    else tile_body<MODE, NW, WRG, BN, 2>(a, t, s_tok);
  } else {
    switch (ncb) {
      case 1: tile_body<MODE, NW, WRG, BN, 1>(a, t, s_tok); break;
      case 2: tile_body<MODE, NW, WRG, BN, 2>(a, t, s_tok); break;
      case 3: tile_body<MODE, NW, WRG, BN, 3>(a, t, s_tok); break;
      case 4: tile_body<MODE, NW, WRG, BN, 4>(a, t, s_tok); break;
      case 5: tile_body<MODE, NW, WRG, BN, 5>(a, t, s_tok); break;
      case 6: tile_body<MODE, NW, WRG, BN, 6>(a, t, s_tok); break;
      case 7: tile_body<MODE, NW, WRG, BN, 7>(a, t, s_tok); break;
      default: tile_body<MODE, NW, WRG, BN, 8>(a, t, s_tok); break;
    }
  }
}

// out[t, 8v..8v+7] = BF16(sum_j w[t, j] * o[expanded_row_idx[t*k + j], 8v..8v+7]), j in
// order, fp32 fused multiply-add.  A workgroup covers 8*kFinThreads columns of one token
// (the token's row indices and weights are the same for the whole wave); each thread owns
// 8 columns and issues the 16-byte loads of up to kFinBatch routed rows before it
// accumulates them, so a wave keeps that many row reads in flight.
constexpr int kFinThreads = 256, kFinBatch = 8;

__global__ __launch_bounds__(kFinThreads) void finalize_kernel(LayerArgs a, int col_blocks) {
  const int64_t t = blockIdx.x / col_blocks;
  const int v = (blockIdx.x % col_blocks) * kFinThreads + threadIdx.x;
  if (v >= a.H / 8) return;
  const int32_t* __restrict__ pos_t = a.expanded_row_idx + t * a.k;
  const uint16_t* __restrict__ w_t = a.route_weights + t * a.k;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < a.k; j0 += kFinBatch) {
    uint4 d[kFinBatch];
    bool ok[kFinBatch];
#pragma unroll
    for (int u = 0; u < kFinBatch; ++u) {
      const int j = j0 + u;
      const int64_t pos = j < a.k ? pos_t[j] : -1;
      ok[u] = pos >= 0;                         // < 0: dropped (expert id out of range)
      d[u] = ok[u] ? reinterpret_cast<const uint4*>(a.o_rows + pos * a.H)[v] : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kFinBatch; ++u) {
      if (!ok[u]) continue;
      const float wt = bf16_to_f32(w_t[j0 + u]);
      const uint32_t dw[4] = {d[u].x, d[u].y, d[u].z, d[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(wt, __uint_as_float(dw[i] << 16), acc[2 * i]);
        acc[2 * i + 1] = fmaf(wt, __uint_as_float(dw[i] & 0xFFFF0000u), acc[2 * i + 1]);
      }
    }
  }
  uint4 o;
  o.x = f32_to_bf16_rne(acc[0]) | (static_cast<uint32_t>(f32_to_bf16_rne(acc[1])) << 16);
  o.y = f32_to_bf16_rne(acc[2]) | (static_cast<uint32_t>(f32_to_bf16_rne(acc[3])) << 16);
  o.z = f32_to_bf16_rne(acc[4]) | (static_cast<uint32_t>(f32_to_bf16_rne(acc[5])) << 16);
  o.w = f32_to_bf16_rne(acc[6]) | (static_cast<uint32_t>(f32_to_bf16_rne(acc[7])) << 16);
  reinterpret_cast<uint4*>(a.out + t * a.H)[v] = o;
}


// Variants: small tiles (up to 32 tokens) run 4 waves x 2 groups (128-row slabs); big
// tiles (up to kBigRows tokens) run kBigNW waves x kBigWRG groups when the slab divides
// the rows, else the 128-row slab.
constexpr int kBigNW = 4, kBigWRG = 2, kBigWPE = 2;

template <int MODE, int NW, int WRG, int BN, int WPE>
static void launch_variant(const LayerArgs& a, int64_t max_tiles, int big, hipStream_t stream) {
  using C = GemmCfg<MODE, NW, WRG, BN>;
  const int rows_total = MODE == 0 ? 2 * a.I : a.H;
  const int64_t grid = round_up(round_up(max_tiles, kTileGroup) * (rows_total / C::kWgRows),
                                kXcds * kXcdRun);
  if (grid > 0)
    grouped_gemm_kernel<MODE, NW, WRG, BN, WPE>
        <<<dim3(static_cast<unsigned>(grid)), dim3(C::kThreads), 0, stream>>>(a, big);
}

template <int MODE>
static hipError_t launch_gemm(const LayerArgs& a, hipStream_t stream) {
  const int rows_total = MODE == 0 ? 2 * a.I : a.H;
  launch_variant<MODE, 4, 2, kSmallRows, 1>(a, a.max_small, 0, stream);
  if (rows_total % GemmCfg<MODE, kBigNW, kBigWRG, kBigRows>::kWgRows == 0)
    launch_variant<MODE, kBigNW, kBigWRG, kBigRows, kBigWPE>(a, a.max_big, 1, stream);
  else
    launch_variant<MODE, 4, 2, kBigRows, 1>(a, a.max_big, 1, stream);
  return hipGetLastError();
}

hipError_t launch_fc1(const LayerArgs& a, hipStream_t stream) { return launch_gemm<0>(a, stream); }
constexpr int64_t kFc2ResidentBigMinRows = 2 * 256 * kBigRows;

hipError_t launch_fc2(const LayerArgs& a, hipStream_t stream) {
  if (!fc2_resident_fits(a)) return launch_gemm<1>(a, stream);
  launch_fc2_resident_small(a, stream);
  // The resident kernel gives each big tile one workgroup; below about two big tiles per
  // CU that leaves the chip idle, and the grouped kernel (tiles x row slabs) is faster.
  if (static_cast<int64_t>(a.T) * a.k >= kFc2ResidentBigMinRows) launch_fc2_resident_big(a, stream);
  else if (a.H % GemmCfg<1, kBigNW, kBigWRG, kBigRows>::kWgRows == 0)
    launch_variant<1, kBigNW, kBigWRG, kBigRows, kBigWPE>(a, a.max_big, 1, stream);
  else
    launch_variant<1, 4, 2, kBigRows, 1>(a, a.max_big, 1, stream);
  return hipGetLastError();
}

hipError_t launch_finalize(const LayerArgs& a, hipStream_t stream) {
  const int col_blocks = (a.H / 8 + kFinThreads - 1) / kFinThreads;
  const int64_t grid = static_cast<int64_t>(a.T) * col_blocks;
  if (grid > 0)
    finalize_kernel<<<dim3(static_cast<unsigned>(grid)), dim3(kFinThreads), 0, stream>>>(a, col_blocks);
  return hipGetLastError();
}

}  // namespace rmoe
