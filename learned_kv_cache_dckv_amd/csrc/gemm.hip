// Transform stages of the DCKV codec on gfx950: bf16 MFMA GEMMs with fp32
// accumulation and fused epilogues.
//
// Source: DCKV digest page ("DCKV: Learned Transform Coding of the Prompt KV
// Cache in Hybrid Language Models"), "How it works":
//   - Transform: one shared basis maps every 6,144-dim row to 2,048
//     coefficients; a small nonlinear correction (one hidden layer of 256
//     GELU units) is added on the synthesis side;
//   - Conditional entropy models: even positions take their code means from
//     the prompt token's input embedding, odd positions also from the decoded
//     coefficients of both neighbours (a 1-D checkerboard, two passes);
//   - first paragraph: keys are taken before RoPE, which is reapplied after
//     decoding.
//
// Every GEMM here is C[m][n] = sum_k A[m][k] * B[n][k] with both operands
// k-contiguous (token rows times weight rows).  One workgroup of 4 wave64s
// computes a 128x128 tile; each wave owns a 64x64 sub-tile as 4x4 blocks of
// v_mfma_f32_16x16x32_bf16.  Operand tiles of 128x64 bf16 are staged through
// LDS, double buffered, with the next tile's global loads in flight while the
// current one feeds the matrix cores.
//
// Epilogues:
//   mean       H E[tok] -> fp32, stored in a 4-row-interleaved layout that the
//              quantiser reads with one 16-byte load per 4 rows
//   quantise   r = (y - mu) / step, q = rint(r), symbols, escapes; even rows
//              first, then odd rows with both neighbours (from LDS); the last
//              odd row of a tile is finished by a small fix-up kernel
//   dequant    yhat = mu + q step in the same two passes -> bf16 yhat_b
//   w1         GELU(exact erf) -> bf16 h_b
//   synthesis  RoPE on key heads (rotate-half) -> bf16 rows
#include <cmath>

#include "dckv_internal.h"

namespace dckv {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kThreads = 256;
constexpr int kLdsStride = kBK + 8;                      // bf16 per staged row (144 B)
constexpr int kStage = (kBM + kBN) * kLdsStride;         // bf16 per stage
constexpr int kTileStride = kBM + 4;                     // floats per column of the epilogue tile
constexpr int kLdsBytes = 2 * kStage * 2 > kBN * kTileStride * 4 ? 2 * kStage * 2 : kBN * kTileStride * 4;
constexpr float kQLimit = 2147483520.0f;                 // largest float below 2^31

__device__ __forceinline__ void set_status(int32_t *st, int code) { atomicCAS(st, 0, code); }

// One read of the status word per workgroup, so that every wave of the
// workgroup takes the same early exit (other workgroups may set it meanwhile).
__device__ __forceinline__ bool wg_stop(const int32_t *st) {
  __shared__ int s_stop;
  if (threadIdx.x == 0) s_stop = *reinterpret_cast<const volatile int32_t *>(st);
  __syncthreads();
  return s_stop != 0;
}

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (finite inputs; NaN kept quiet)
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Operand rows of one tile: 4 rows per thread (tid/8 + 32u), two k-ranges.
struct Src {
  const uint16_t *p0[4];
  const uint16_t *p1[4];
  int split;  // k-tiles [0, split) from p0, the rest from p1
};

__device__ __forceinline__ uint4 ld_chunk(const Src &s, int u, int kt, int kc) {
  const uint16_t *p = kt < s.split ? s.p0[u] + kt * kBK : s.p1[u] + (kt - s.split) * kBK;
  return *reinterpret_cast<const uint4 *>(p + kc * 8);
}

__device__ __forceinline__ void mainloop(const Src &A, const Src &B, int KT, f32x4 (&acc)[4][4], uint16_t *lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = tid >> 3, kc = tid & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint4 ra[4], rb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    ra[u] = ld_chunk(A, u, 0, kc);
    rb[u] = ld_chunk(B, u, 0, kc);
  }
  {
    uint16_t *sa = lds, *sb = lds + kBM * kLdsStride;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      *reinterpret_cast<uint4 *>(sa + (lr + 32 * u) * kLdsStride + kc * 8) = ra[u];
      *reinterpret_cast<uint4 *>(sb + (lr + 32 * u) * kLdsStride + kc * 8) = rb[u];
    }
  }
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        ra[u] = ld_chunk(A, u, kt + 1, kc);
        rb[u] = ld_chunk(B, u, kt + 1, kc);
      }
    }
    const uint16_t *sa = lds + cur * kStage;
    const uint16_t *sb = sa + kBM * kLdsStride;
#pragma unroll
    for (int ks = 0; ks < kBK / 32; ++ks) {
      bf16x8 af[4], bfr[4];
      const int ko = ks * 32 + (lane >> 4) * 8;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        af[mb] = *reinterpret_cast<const bf16x8 *>(sa + (wm * 64 + mb * 16 + (lane & 15)) * kLdsStride + ko);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        bfr[nb] = *reinterpret_cast<const bf16x8 *>(sb + (wn * 64 + nb * 16 + (lane & 15)) * kLdsStride + ko);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
    }
    if (kt + 1 < KT) {
      uint16_t *da = lds + (cur ^ 1) * kStage, *db = da + kBM * kLdsStride;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        *reinterpret_cast<uint4 *>(da + (lr + 32 * u) * kLdsStride + kc * 8) = ra[u];
        *reinterpret_cast<uint4 *>(db + (lr + 32 * u) * kLdsStride + kc * 8) = rb[u];
      }
    }
    __syncthreads();
  }
}

// Accumulators -> LDS tile, column-major: tile[n * kTileStride + m].
// Lane l of a 16x16 block holds rows 4*(l/16) .. +3 of column l%16.
__device__ __forceinline__ void acc_to_tile(const f32x4 (&acc)[4][4], float *tile) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int col = wn * 64 + nb * 16 + (lane & 15);
      const int row = wm * 64 + mb * 16 + (lane >> 4) * 4;
      *reinterpret_cast<f32x4 *>(tile + col * kTileStride + row) = acc[mb][nb];
    }
}

// ---------------------------------------------------------------------------
// operand row pointers (per thread: rows tid/8 + 32u of the tile)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int clamp_tok(const int32_t *tok, int64_t t, int vocab, int32_t *status) {
  int v = tok[t];
  if (v < 0 || v >= vocab) {
    set_status(status, DCKV_EINVAL);
    v = 0;
  }
  return v;
}

// ---------------------------------------------------------------------------
// encode: mean GEMM  m[j][r] = sum_k E[tok_{j+kh}][k] H[act[r]][k]
// ---------------------------------------------------------------------------
struct MeanEncP {
  const uint16_t *E, *H;
  const int32_t *tok, *act;
  float *mean;  // [NM/4][Ca4][4]
  int64_t N, Ca4;
  int keep_head, vocab;
  int32_t *status;
};

__global__ __launch_bounds__(kThreads) void k_mean_enc(MeanEncP P) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[kLdsBytes];
  uint16_t *lds = reinterpret_cast<uint16_t *>(lds_raw);
  if (wg_stop(P.status)) return;
  const int64_t m0 = (int64_t)blockIdx.y * kBM;
  const int n0 = blockIdx.x * kBN;
  const int lr = threadIdx.x >> 3;
  Src A, B;
  A.split = B.split = kEmb / kBK;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t j = min<int64_t>(m0 + lr + 32 * u, P.N - 1);
    A.p0[u] = A.p1[u] = P.E + (size_t)clamp_tok(P.tok, P.keep_head + j, P.vocab, P.status) * kEmb;
    B.p0[u] = B.p1[u] = P.H + (size_t)P.act[n0 + lr + 32 * u] * kEmb;
  }
  f32x4 acc[4][4];
  mainloop(A, B, kEmb / kBK, acc, lds);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int64_t row = m0 + wm * 64 + mb * 16 + (lane >> 4) * 4;
      const int64_t col = n0 + wn * 64 + nb * 16 + (lane & 15);
      *reinterpret_cast<f32x4 *>(P.mean + ((row >> 2) * P.Ca4 + col) * 4) = acc[mb][nb];
    }
}

// ---------------------------------------------------------------------------
// encode: analysis GEMM + quantiser (two checkerboard passes)
// ---------------------------------------------------------------------------
struct QuantP {
  const uint16_t *rows, *A;
  const int32_t *act;
  const float *step, *nbr, *mean;
  uint32_t *sym32;
  uint32_t *esc_raw;   // {flat, q}
  uint8_t *ws;
  float *halo_a, *halo_b;
  int64_t N, N256, Ca4, esc_cap;
  int Ca, keep_head, C;
  int32_t *status;
};

__device__ __forceinline__ uint32_t quant_one(float d, float step, int64_t j, int r, const QuantP &P, bool &bad,
                                              float &qf) {
  if (!isfinite(d)) {
    bad = true;
    qf = 0.f;
    return 127u;
  }
  qf = fminf(fmaxf(rintf(d / step), -kQLimit), kQLimit);
  const int qi = (int)qf;
  if (qi >= -127 && qi <= 127) return (uint32_t)(qi + 127);
  Ctrl *ct = reinterpret_cast<Ctrl *>(P.ws);
  const uint32_t idx = atomicAdd(&ct->n_esc, 1u);
  if ((int64_t)idx < P.esc_cap) {
    P.esc_raw[2 * idx] = (uint32_t)(j * P.Ca + r);
    P.esc_raw[2 * idx + 1] = (uint32_t)qi;
  }
  return (uint32_t)kEsc;
}

__global__ __launch_bounds__(kThreads) void k_analysis_quant(QuantP P) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[kLdsBytes];
  uint16_t *lds = reinterpret_cast<uint16_t *>(lds_raw);
  if (wg_stop(P.status)) return;
  const int64_t m0 = (int64_t)blockIdx.y * kBM;
  const int n0 = blockIdx.x * kBN;
  const int lr = threadIdx.x >> 3;
  Src A, B;
  A.split = B.split = kD / kBK;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t j = min<int64_t>(m0 + lr + 32 * u, P.N - 1);
    A.p0[u] = A.p1[u] = P.rows + (size_t)(P.keep_head + j) * kD;
    B.p0[u] = B.p1[u] = P.A + (size_t)P.act[n0 + lr + 32 * u] * kD;
  }
  f32x4 acc[4][4];
  mainloop(A, B, kD / kBK, acc, lds);
  float *tile = reinterpret_cast<float *>(lds_raw);
  acc_to_tile(acc, tile);
  __syncthreads();

  const int col = threadIdx.x & 127, half = threadIdx.x >> 7;
  const int r = n0 + col;
  const bool rv = r < P.Ca;
  const int c = P.act[r];
  const float step = P.step[c], a = P.nbr[c];
  float *tc = tile + col * kTileStride;
  const int64_t mt = blockIdx.y;
  uint32_t symw[16];
  bool bad = false;
  // pass 1: even rows, mu = H E[tok]
#pragma unroll 4
  for (int qd = 0; qd < 16; ++qd) {
    const int rq = half * 64 + qd * 4;
    const int64_t j0 = m0 + rq;
    const f32x4 mm = *reinterpret_cast<const f32x4 *>(P.mean + ((j0 >> 2) * P.Ca4 + r) * 4);
    uint32_t w = 0xFFFFFFFFu;
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      const int64_t j = j0 + e;
      if (j < P.N && rv) {
        float qf;
        const uint32_t s = quant_one(tc[rq + e] - mm[e], step, j, r, P, bad, qf);
        tc[rq + e] = mm[e] + qf * step;
        w = (w & ~(0xFFu << (8 * e))) | (s << (8 * e));
      } else {
        tc[rq + e] = 0.f;  // a missing right neighbour counts as zero
      }
    }
    symw[qd] = w;
  }
  __syncthreads();
  if (half == 0 && rv) P.halo_b[mt * P.C + r] = tc[0];
  // pass 2: odd rows, mu = H E[tok] + a (yhat_{j-1} + yhat_{j+1})
#pragma unroll 4
  for (int qd = 0; qd < 16; ++qd) {
    const int rq = half * 64 + qd * 4;
    const int64_t j0 = m0 + rq;
    const f32x4 mm = *reinterpret_cast<const f32x4 *>(P.mean + ((j0 >> 2) * P.Ca4 + r) * 4);
    uint32_t w = symw[qd];
#pragma unroll
    for (int e = 1; e < 4; e += 2) {
      const int row = rq + e;
      const int64_t j = j0 + e;
      if (!(j < P.N && rv)) continue;
      const float prev = tc[row - 1];
      uint32_t s;
      if (row == kBM - 1 && j + 1 < P.N) {
        P.halo_a[mt * P.C + r] = tc[row] - mm[e] - a * prev;  // finished by the fix-up
        s = 0u;
      } else {
        const float next = row + 1 < kBM ? tc[row + 1] : 0.f;
        const float mu = mm[e] + a * (prev + next);
        float qf;
        s = quant_one(tc[row] - mu, step, j, r, P, bad, qf);
      }
      w = (w & ~(0xFFu << (8 * e))) | (s << (8 * e));
    }
    if (j0 < P.N && rv) P.sym32[((size_t)(r >> 6) * (P.N256 / 4) + (j0 >> 2)) * 64 + (r & 63)] = w;
  }
  if (bad) set_status(P.status, DCKV_EINVAL);
}

// last odd row of every row tile whose right neighbour is in the next tile
__global__ void k_encode_fixup(QuantP P, int64_t n_fix) {
  if (*P.status != 0) return;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_fix * P.Ca) return;
  const int64_t mt = i / P.Ca;
  const int r = (int)(i - mt * P.Ca);
  const int64_t j = (mt + 1) * kBM - 1;
  const int c = P.act[r];
  const float step = P.step[c], a = P.nbr[c];
  const float d = P.halo_a[mt * P.C + r] - a * P.halo_b[(mt + 1) * P.C + r];
  bool bad = false;
  float qf;
  const uint32_t s = quant_one(d, step, j, r, P, bad, qf);
  uint8_t *sym8 = reinterpret_cast<uint8_t *>(P.sym32);
  sym8[(((size_t)(r >> 6) * (P.N256 / 4) + (j >> 2)) * 64 + (r & 63)) * 4 + (j & 3)] = (uint8_t)s;
  if (bad) set_status(P.status, DCKV_EINVAL);
}

// ---------------------------------------------------------------------------
// decode: mean GEMM over all components + two dequantisation passes
// ---------------------------------------------------------------------------
struct DeqP {
  const uint16_t *E, *H;
  const int32_t *tok, *rank;
  const float *step, *nbr;
  const uint32_t *sym32;
  const uint8_t *stream;
  const uint8_t *ws;
  uint16_t *yhat_b;  // [NM][C]
  float *halo_a, *halo_b;
  int64_t N, N256;
  int Ca, keep_head, vocab;
  int32_t *status;
};

__device__ __forceinline__ int esc_code(const DeqP &P, uint32_t flat) {
  const Ctrl *ct = reinterpret_cast<const Ctrl *>(P.ws);
  const uint32_t *esc = reinterpret_cast<const uint32_t *>(P.stream + ct->esc_off);
  uint32_t lo = 0, hi = ct->n_esc;
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    if (esc[2 * mid] < flat) lo = mid + 1; else hi = mid;
  }
  if (lo < ct->n_esc && esc[2 * lo] == flat) return (int)esc[2 * lo + 1];
  set_status(const_cast<int32_t *>(P.status), DCKV_ECORRUPT);
  return 0;
}

__device__ __forceinline__ float code_of(const DeqP &P, uint32_t w, int e, int64_t j, int r) {
  const uint32_t s = (w >> (8 * e)) & 0xFFu;
  if (s != (uint32_t)kEsc) return (float)((int)s - 127);
  return (float)esc_code(P, (uint32_t)(j * P.Ca + r));
}

// row-major bf16 store of a 128x128 LDS tile (column-major floats)
template <class F>
__device__ __forceinline__ void store_tile_rows(const float *tile, uint16_t *out, int64_t ld, int64_t m0, int n0,
                                                int64_t rows_valid, F &&fn) {
  const int t = threadIdx.x;
  const int cg = t & 15;
  for (int rr = t >> 4; rr < kBM; rr += kThreads / 16) {
    if (m0 + rr >= rows_valid) break;
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = f2bf(fn(tile[(cg * 8 + e) * kTileStride + rr]));
    uint4 pk;
    pk.x = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
    pk.y = (uint32_t)v[2] | ((uint32_t)v[3] << 16);
    pk.z = (uint32_t)v[4] | ((uint32_t)v[5] << 16);
    pk.w = (uint32_t)v[6] | ((uint32_t)v[7] << 16);
    *reinterpret_cast<uint4 *>(out + (size_t)(m0 + rr) * ld + n0 + cg * 8) = pk;
  }
}

__global__ __launch_bounds__(kThreads) void k_dequant(DeqP P) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[kLdsBytes];
  uint16_t *lds = reinterpret_cast<uint16_t *>(lds_raw);
  if (wg_stop(P.status)) return;
  const int64_t m0 = (int64_t)blockIdx.y * kBM;
  const int n0 = blockIdx.x * kBN;
  const int lr = threadIdx.x >> 3;
  Src A, B;
  A.split = B.split = kEmb / kBK;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t j = min<int64_t>(m0 + lr + 32 * u, P.N - 1);
    A.p0[u] = A.p1[u] = P.E + (size_t)clamp_tok(P.tok, P.keep_head + j, P.vocab, P.status) * kEmb;
    B.p0[u] = B.p1[u] = P.H + (size_t)(n0 + lr + 32 * u) * kEmb;
  }
  f32x4 acc[4][4];
  mainloop(A, B, kEmb / kBK, acc, lds);
  float *tile = reinterpret_cast<float *>(lds_raw);
  acc_to_tile(acc, tile);
  __syncthreads();

  const int col = threadIdx.x & 127, half = threadIdx.x >> 7;
  const int c = n0 + col;
  const int r = P.rank[c];
  const float step = P.step[c], a = P.nbr[c];
  float *tc = tile + col * kTileStride;
  const int64_t mt = blockIdx.y;
  uint32_t symw[16];
#pragma unroll 4
  for (int qd = 0; qd < 16; ++qd) {
    const int rq = half * 64 + qd * 4;
    const int64_t j0 = m0 + rq;
    const uint32_t w = (r >= 0 && j0 < P.N)
                           ? P.sym32[((size_t)(r >> 6) * (P.N256 / 4) + (j0 >> 2)) * 64 + (r & 63)]
                           : 0x7F7F7F7Fu;  // code 0
    symw[qd] = w;
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      const int64_t j = j0 + e;
      if (j < P.N) {
        const float q = r >= 0 ? code_of(P, w, e, j, r) : 0.f;
        tc[rq + e] = tc[rq + e] + q * step;
      } else {
        tc[rq + e] = 0.f;
      }
    }
  }
  __syncthreads();
  if (half == 0) P.halo_b[mt * kC + c] = tc[0];
  // odd rows read only even rows, so they may be overwritten in place
#pragma unroll 4
  for (int qd = 0; qd < 16; ++qd) {
    const int rq = half * 64 + qd * 4;
    const int64_t j0 = m0 + rq;
    const uint32_t w = symw[qd];
#pragma unroll
    for (int e = 1; e < 4; e += 2) {
      const int row = rq + e;
      const int64_t j = j0 + e;
      if (j >= P.N) {
        tc[row] = 0.f;
        continue;
      }
      const float q = r >= 0 ? code_of(P, w, e, j, r) : 0.f;
      const float prev = tc[row - 1];
      if (row == kBM - 1 && j + 1 < P.N) {
        P.halo_a[mt * kC + c] = tc[row] + a * prev + q * step;  // finished by the fix-up
      } else {
        const float next = row + 1 < kBM ? tc[row + 1] : 0.f;
        tc[row] = tc[row] + a * (prev + next) + q * step;
      }
    }
  }
  __syncthreads();
  store_tile_rows(tile, P.yhat_b, kC, m0, n0, P.N, [](float v) { return v; });
}

__global__ void k_decode_fixup(DeqP P, int64_t n_fix) {
  if (*P.status != 0) return;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_fix * kC) return;
  const int64_t mt = i / kC;
  const int c = (int)(i - mt * kC);
  const int64_t j = (mt + 1) * kBM - 1;
  const float y = P.halo_a[mt * kC + c] + P.nbr[c] * P.halo_b[(mt + 1) * kC + c];
  P.yhat_b[(size_t)j * kC + c] = f2bf(y);
}

// ---------------------------------------------------------------------------
// decode: correction hidden layer h = GELU(W1 yhat_b)
// ---------------------------------------------------------------------------
struct W1P {
  const uint16_t *yhat_b, *W1;
  uint16_t *h_b;  // [NM][256]
  int64_t N;
  const int32_t *status;
};

__global__ __launch_bounds__(kThreads) void k_w1(W1P P) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[kLdsBytes];
  uint16_t *lds = reinterpret_cast<uint16_t *>(lds_raw);
  if (wg_stop(P.status)) return;
  const int64_t m0 = (int64_t)blockIdx.y * kBM;
  const int n0 = blockIdx.x * kBN;
  const int lr = threadIdx.x >> 3;
  Src A, B;
  A.split = B.split = kC / kBK;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    A.p0[u] = A.p1[u] = P.yhat_b + (size_t)(m0 + lr + 32 * u) * kC;
    B.p0[u] = B.p1[u] = P.W1 + (size_t)(n0 + lr + 32 * u) * kC;
  }
  f32x4 acc[4][4];
  mainloop(A, B, kC / kBK, acc, lds);
  float *tile = reinterpret_cast<float *>(lds_raw);
  acc_to_tile(acc, tile);
  __syncthreads();
  store_tile_rows(tile, P.h_b, kHid, m0, n0, P.N,
                  [](float u) { return 0.5f * u * (1.0f + erff(u * 0.70710678118654752f)); });
}

// ---------------------------------------------------------------------------
// decode: synthesis xhat = S yhat_b + W2 h_b with RoPE on key heads
// ---------------------------------------------------------------------------
struct SynP {
  const uint16_t *yhat_b, *h_b, *S, *W2;
  const float2 *rope_lo, *rope_hi;  // [256][128], [ceil(T/256)][128]: (cos, sin)
  uint16_t *out;                     // rows_out [T][D]
  int64_t N;
  int keep_head;
  const int32_t *status;
};

// GEMM column n of tile nt -> output dim.  Tile nt covers head nt/2 (256
// dims) and the pair-aligned halves d0 + [0,64) and d0 + 128 + [0,64), with
// d0 = 64 * (nt % 2), so a rotate-half pair (d, d+128) stays in one tile.
__device__ __forceinline__ int syn_dim(int nt, int n) {
  return (nt >> 1) * kHeadDim + (nt & 1) * 64 + n + (n >= 64 ? 64 : 0);
}

__global__ __launch_bounds__(kThreads) void k_synthesis(SynP P) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[kLdsBytes];
  uint16_t *lds = reinterpret_cast<uint16_t *>(lds_raw);
  if (wg_stop(P.status)) return;
  const int64_t m0 = (int64_t)blockIdx.y * kBM;
  const int nt = blockIdx.x;
  const int lr = threadIdx.x >> 3;
  Src A, B;
  A.split = B.split = kC / kBK;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t j = m0 + lr + 32 * u;
    A.p0[u] = P.yhat_b + (size_t)j * kC;
    A.p1[u] = P.h_b + (size_t)j * kHid;
    const int dim = syn_dim(nt, lr + 32 * u);
    B.p0[u] = P.S + (size_t)dim * kC;
    B.p1[u] = P.W2 + (size_t)dim * kHid;
  }
  f32x4 acc[4][4];
  mainloop(A, B, (kC + kHid) / kBK, acc, lds);
  float *tile = reinterpret_cast<float *>(lds_raw);
  acc_to_tile(acc, tile);
  __syncthreads();

  const int head = nt >> 1;
  const bool is_key = (head & 3) < 2;  // per layer: 2 key heads then 2 value heads
  const int d0 = (nt & 1) * 64;
  const int t = threadIdx.x;
  const int pg = t & 7;  // 8 pairs per thread
  for (int rr = t >> 3; rr < kBM; rr += kThreads / 8) {
    const int64_t j = m0 + rr;
    if (j >= P.N) break;
    const int64_t pos = P.keep_head + j;
    uint16_t lo_v[8], hi_v[8];
    if (is_key) {
      const float2 *tl = P.rope_lo + (size_t)(pos & 255) * kHalf + d0 + pg * 8;
      const float2 *th = P.rope_hi + (size_t)(pos >> 8) * kHalf + d0 + pg * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 a = tl[e], b = th[e];
        const float cs = b.x * a.x - b.y * a.y;
        const float sn = b.y * a.x + b.x * a.y;
        const float x0 = tile[(pg * 8 + e) * kTileStride + rr];
        const float x1 = tile[(64 + pg * 8 + e) * kTileStride + rr];
        lo_v[e] = f2bf(x0 * cs - x1 * sn);
        hi_v[e] = f2bf(x1 * cs + x0 * sn);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        lo_v[e] = f2bf(tile[(pg * 8 + e) * kTileStride + rr]);
        hi_v[e] = f2bf(tile[(64 + pg * 8 + e) * kTileStride + rr]);
      }
    }
    uint16_t *o = P.out + (size_t)pos * kD + head * kHeadDim + d0 + pg * 8;
    uint4 a4, b4;
    a4.x = lo_v[0] | ((uint32_t)lo_v[1] << 16); a4.y = lo_v[2] | ((uint32_t)lo_v[3] << 16);
    a4.z = lo_v[4] | ((uint32_t)lo_v[5] << 16); a4.w = lo_v[6] | ((uint32_t)lo_v[7] << 16);
    b4.x = hi_v[0] | ((uint32_t)hi_v[1] << 16); b4.y = hi_v[2] | ((uint32_t)hi_v[3] << 16);
    b4.z = hi_v[4] | ((uint32_t)hi_v[5] << 16); b4.w = hi_v[6] | ((uint32_t)hi_v[7] << 16);
    *reinterpret_cast<uint4 *>(o) = a4;
    *reinterpret_cast<uint4 *>(o + kHalf) = b4;
  }
}

// ---------------------------------------------------------------------------
// RoPE angle tables: cos/sin of u*w_i (u < 256) and of 256*v*w_i, in float64
// ---------------------------------------------------------------------------
__global__ void k_rope_tables(const double *omega, float2 *lo, float2 *hi, int64_t n_hi) {
  const int64_t n = (256 + n_hi) * kHalf;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t u = i / kHalf;
    const int k = (int)(i - u * kHalf);
    double ang;
    float2 *dst;
    if (u < 256) {
      ang = (double)u * omega[k];
      dst = lo + u * kHalf + k;
    } else {
      ang = (double)((u - 256) * 256) * omega[k];
      dst = hi + (u - 256) * kHalf + k;
    }
    double s, c;
    sincos(ang, &s, &c);
    *dst = make_float2((float)c, (float)s);
  }
}

// kept rows: RoPE on key columns of the verbatim rows in the stream
__global__ void k_kept_rope(const uint8_t *stream, const float2 *lo, const float2 *hi, uint16_t *out,
                            int64_t n_kept, int64_t head_n, int64_t tail_pos0, const int32_t *status) {
  if (*status != 0) return;
  const int64_t k = blockIdx.x;
  if (k >= n_kept) return;
  const int64_t pos = k < head_n ? k : tail_pos0 + (k - head_n);
  const uint16_t *src = reinterpret_cast<const uint16_t *>(stream + kHeaderBytes) + (size_t)k * kD;
  uint16_t *dst = out + (size_t)pos * kD;
  for (int i = threadIdx.x; i < kD / 2; i += blockDim.x) {
    // i enumerates (head, d) with d < 128: the pair (d, d + 128) of every head
    const int head = i / kHalf, d = i % kHalf;
    const int base = head * kHeadDim;
    const float x0 = bf2f(src[base + d]), x1 = bf2f(src[base + d + kHalf]);
    if ((head & 3) < 2) {
      const float2 a = lo[(size_t)(pos & 255) * kHalf + d], b = hi[(size_t)(pos >> 8) * kHalf + d];
      const float cs = b.x * a.x - b.y * a.y;
      const float sn = b.y * a.x + b.x * a.y;
      dst[base + d] = f2bf(x0 * cs - x1 * sn);
      dst[base + d + kHalf] = f2bf(x1 * cs + x0 * sn);
    } else {
      dst[base + d] = src[base + d];
      dst[base + d + kHalf] = src[base + d + kHalf];
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
void launch_mean_gemm(const EncodeArgs &a) {
  if (a.g.N == 0 || a.p->C_a == 0) return;
  MeanEncP P;
  P.E = a.p->E;
  P.H = a.p->H;
  P.tok = a.tok;
  P.act = a.p->dev.act;
  P.mean = reinterpret_cast<float *>(a.ws + a.l.mean);
  P.N = a.g.N;
  P.Ca4 = a.g.Ca4;
  P.keep_head = a.p->keep_head;
  P.vocab = a.p->vocab;
  P.status = a.status;
  dim3 grid((unsigned)(a.g.Ca4 / kBN), (unsigned)a.g.n_mtiles);
  KernelTimer tm("mean_gemm", a.s);
  hipLaunchKernelGGL(k_mean_enc, grid, dim3(kThreads), 0, a.s, P);
}

static QuantP quant_params(const EncodeArgs &a) {
  QuantP P;
  P.rows = a.rows;
  P.A = a.p->A;
  P.act = a.p->dev.act;
  P.step = a.p->dev.step;
  P.nbr = a.p->dev.nbr;
  P.mean = reinterpret_cast<const float *>(a.ws + a.l.mean);
  P.sym32 = reinterpret_cast<uint32_t *>(a.ws + a.l.sym);
  P.esc_raw = reinterpret_cast<uint32_t *>(a.ws + a.l.esc_raw);
  P.ws = a.ws;
  P.halo_a = reinterpret_cast<float *>(a.ws + a.l.halo_a);
  P.halo_b = reinterpret_cast<float *>(a.ws + a.l.halo_b);
  P.N = a.g.N;
  P.N256 = a.g.N256;
  P.Ca4 = a.g.Ca4;
  P.esc_cap = a.g.esc_cap;
  P.Ca = a.p->C_a;
  P.keep_head = a.p->keep_head;
  P.C = a.p->C;
  P.status = a.status;
  return P;
}

void launch_analysis_gemm(const EncodeArgs &a) {
  if (a.g.N == 0 || a.p->C_a == 0) return;
  QuantP P = quant_params(a);
  dim3 grid((unsigned)(a.g.Ca4 / kBN), (unsigned)a.g.n_mtiles);
  KernelTimer tm("analysis_gemm", a.s);
  hipLaunchKernelGGL(k_analysis_quant, grid, dim3(kThreads), 0, a.s, P);
}

void launch_encode_fixup(const EncodeArgs &a) {
  if (a.g.N == 0 || a.p->C_a == 0) return;
  const int64_t n_fix = (a.g.N - 1) / kBM;  // tiles t with (t+1)*BM < N
  if (n_fix <= 0) return;
  QuantP P = quant_params(a);
  const int64_t work = n_fix * a.p->C_a;
  KernelTimer tm("fixup", a.s);
  hipLaunchKernelGGL(k_encode_fixup, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, a.s, P, n_fix);
}

void launch_rope_tables(const DecodeArgs &a) {
  const int64_t n = (256 + a.g.rope_hi) * kHalf;
  hipLaunchKernelGGL(k_rope_tables, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 4096)), dim3(256), 0, a.s,
                     a.p->dev.omega, reinterpret_cast<float2 *>(a.ws + a.l.rope_lo),
                     reinterpret_cast<float2 *>(a.ws + a.l.rope_hi), a.g.rope_hi);
}

static DeqP deq_params(const DecodeArgs &a) {
  DeqP P;
  P.E = a.p->E;
  P.H = a.p->H;
  P.tok = a.tok;
  P.rank = a.p->dev.rank;
  P.step = a.p->dev.step;
  P.nbr = a.p->dev.nbr;
  P.sym32 = reinterpret_cast<const uint32_t *>(a.ws + a.l.sym);
  P.stream = a.stream;
  P.ws = a.ws;
  P.yhat_b = reinterpret_cast<uint16_t *>(a.ws + a.l.yhat_b);
  P.halo_a = reinterpret_cast<float *>(a.ws + a.l.halo_a);
  P.halo_b = reinterpret_cast<float *>(a.ws + a.l.halo_b);
  P.N = a.g.N;
  P.N256 = a.g.N256;
  P.Ca = a.p->C_a;
  P.keep_head = a.p->keep_head;
  P.vocab = a.p->vocab;
  P.status = a.status;
  return P;
}

void launch_dequant_gemm(const DecodeArgs &a) {
  if (a.g.N == 0) return;
  DeqP P = deq_params(a);
  dim3 grid((unsigned)(kC / kBN), (unsigned)a.g.n_mtiles);
  KernelTimer tm("dequant_gemm", a.s);
  hipLaunchKernelGGL(k_dequant, grid, dim3(kThreads), 0, a.s, P);
}

void launch_decode_fixup(const DecodeArgs &a) {
  if (a.g.N == 0) return;
  const int64_t n_fix = (a.g.N - 1) / kBM;
  if (n_fix <= 0) return;
  DeqP P = deq_params(a);
  const int64_t work = n_fix * kC;
  KernelTimer tm("fixup", a.s);
  hipLaunchKernelGGL(k_decode_fixup, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, a.s, P, n_fix);
}

void launch_w1_gemm(const DecodeArgs &a) {
  if (a.g.N == 0) return;
  W1P P;
  P.yhat_b = reinterpret_cast<const uint16_t *>(a.ws + a.l.yhat_b);
  P.W1 = a.p->W1;
  P.h_b = reinterpret_cast<uint16_t *>(a.ws + a.l.h_b);
  P.N = a.g.N;
  P.status = a.status;
  dim3 grid((unsigned)(kHid / kBN), (unsigned)a.g.n_mtiles);
  KernelTimer tm("w1_gemm", a.s);
  hipLaunchKernelGGL(k_w1, grid, dim3(kThreads), 0, a.s, P);
}

void launch_synthesis_gemm(const DecodeArgs &a) {
  if (a.g.N == 0) return;
  SynP P;
  P.yhat_b = reinterpret_cast<const uint16_t *>(a.ws + a.l.yhat_b);
  P.h_b = reinterpret_cast<const uint16_t *>(a.ws + a.l.h_b);
  P.S = a.p->S;
  P.W2 = a.p->W2;
  P.rope_lo = reinterpret_cast<const float2 *>(a.ws + a.l.rope_lo);
  P.rope_hi = reinterpret_cast<const float2 *>(a.ws + a.l.rope_hi);
  P.out = a.rows_out;
  P.N = a.g.N;
  P.keep_head = a.p->keep_head;
  P.status = a.status;
  dim3 grid((unsigned)(kD / kBN), (unsigned)a.g.n_mtiles);
  KernelTimer tm("synthesis_gemm", a.s);
  hipLaunchKernelGGL(k_synthesis, grid, dim3(kThreads), 0, a.s, P);
}

void launch_kept_rope(const DecodeArgs &a) {
  if (a.g.n_kept == 0) return;
  const int64_t head_n = std::min<int64_t>(a.p->keep_head, a.g.T);
  const int64_t tail_pos0 = a.p->keep_head + a.g.N;
  hipLaunchKernelGGL(k_kept_rope, dim3((unsigned)a.g.n_kept), dim3(256), 0, a.s, a.stream,
                     reinterpret_cast<const float2 *>(a.ws + a.l.rope_lo),
                     reinterpret_cast<const float2 *>(a.ws + a.l.rope_hi), a.rows_out, a.g.n_kept, head_n,
                     tail_pos0, a.status);
}

}  // namespace dckv
