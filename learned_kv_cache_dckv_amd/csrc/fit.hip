// Closed-form fit of the conditional models to a trained codec, on gfx950.
//
// Source: DCKV digest page ("DCKV: Learned Transform Coding of the Prompt KV
// Cache in Hybrid Language Models"), Evidence: the conditional models can be
// fitted in closed form to an already-trained codec.  The estimators (the
// page names none) are the plainest closed forms for the models of "How it
// works", Conditional entropy models:
//   - y_j = A x_j over n consecutive calibration rows, e_j = E[tok_j];
//   - mean head by ridge least squares, H^T = (E^T E + lam n I)^-1 E^T Y;
//   - with m_j = bf16(H) e_j: for each component, a = sum r s / sum s^2 over
//     the odd rows (r = y - m, s = y_{j-1} + y_{j+1}, y_n = 0);
//   - b = mean |y - mu| over all rows (mu = m, plus a s on odd rows).
//
// GPU steps: the three products with a 2,048-wide inner or outer dimension
// (Y = X A^T; G = E^T E; R = E^T Y, Y split into two bf16 halves so that the
// product keeps 16 mantissa bits; M = E[tok] bf16(H)^T) run on the bf16 MFMA
// GEMM of gemm.hip with fp32 accumulation.  The solve is a blocked Cholesky
// factorisation (64 x 64 blocks, fp32) followed by blocked forward and
// backward substitution over the 2,048 right-hand sides; the per-component
// fits are column reductions.
#include <cmath>

#include "dckv_internal.h"

namespace dckv {
namespace {

constexpr int kNB = 64;            // Cholesky block
constexpr int kNBlk = kEmb / kNB;  // 32 block rows

__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__global__ void k_fit_clear_status(int32_t *status) { *status = 0; }

// The transposes below move 64 x 64 tiles through LDS with 8- or 16-byte
// accesses: 16 threads cover one 64-element row, 16 rows per pass.

// Et[e][j] = E[tok_j][e] for j < n, 0 for n <= j < n_pad (bf16, transposed);
// an id outside [0, vocab) sets EINVAL and reads as 0; tokc receives the
// checked ids (row indices of the later gather GEMM)
__global__ __launch_bounds__(256) void k_fit_gather_t(const uint16_t *E, const int32_t *tok, int64_t n,
                                                      int64_t n_pad, int vocab, uint16_t *Et, int32_t *tokc,
                                                      int32_t *status) {
  __shared__ uint16_t t[64][72];
  const int64_t j0 = (int64_t)blockIdx.x * 64;
  const int e0 = blockIdx.y * 64;
  const int q = threadIdx.x & 15, r = threadIdx.x >> 4;
  for (int p = 0; p < 4; ++p) {
    const int jr = r + 16 * p;
    const int64_t j = j0 + jr;
    uint2 v = make_uint2(0u, 0u);
    if (j < n) {
      int id = tok[j];
      if (id < 0 || id >= vocab) {
        atomicCAS(status, 0, DCKV_EINVAL);
        id = 0;
      }
      v = *reinterpret_cast<const uint2 *>(E + (size_t)id * kEmb + e0 + 4 * q);
      if (blockIdx.y == 0 && q == 0) tokc[j] = id;
    }
    *reinterpret_cast<uint2 *>(&t[jr][4 * q]) = v;
  }
  __syncthreads();
  for (int p = 0; p < 4; ++p) {
    const int er = r + 16 * p;
    const uint32_t a = (uint32_t)t[4 * q][er] | ((uint32_t)t[4 * q + 1][er] << 16);
    const uint32_t b = (uint32_t)t[4 * q + 2][er] | ((uint32_t)t[4 * q + 3][er] << 16);
    *reinterpret_cast<uint2 *>(Et + (size_t)(e0 + er) * n_pad + j0 + 4 * q) = make_uint2(a, b);
  }
}

// Yt_hi[c][j] = bf16(Y[j][c]), Yt_lo[c][j] = bf16(Y[j][c] - Yt_hi), zero for j >= n
__global__ __launch_bounds__(256) void k_fit_split_t(const float *Y, int64_t n, int64_t n_pad, uint16_t *hi,
                                                     uint16_t *lo) {
  __shared__ float t[64][68];
  const int64_t j0 = (int64_t)blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  const int q = threadIdx.x & 15, r = threadIdx.x >> 4;
  for (int p = 0; p < 4; ++p) {
    const int jr = r + 16 * p;
    const int64_t j = j0 + jr;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (j < n) v = *reinterpret_cast<const float4 *>(Y + (size_t)j * kC + c0 + 4 * q);
    *reinterpret_cast<float4 *>(&t[jr][4 * q]) = v;
  }
  __syncthreads();
  for (int p = 0; p < 4; ++p) {
    const int cr = r + 16 * p;
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float y = t[4 * q + i][cr];
      h[i] = f2bf(y);
      l[i] = f2bf(y - bf2f((uint16_t)h[i]));
    }
    const size_t o = (size_t)(c0 + cr) * n_pad + j0 + 4 * q;
    *reinterpret_cast<uint2 *>(hi + o) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    *reinterpret_cast<uint2 *>(lo + o) = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
  }
}

// G += v I; dg keeps the diagonal for the pivot test
__global__ void k_fit_add_diag(float *G, float v, float *dg) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < kEmb) {
    const float d = G[(size_t)i * kEmb + i] + v;
    G[(size_t)i * kEmb + i] = d;
    dg[i] = d;
  }
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Unblocked Cholesky of diagonal block k (lower, in place; the block's upper
// triangle is zeroed, so later kernels read it as L_kk), then its inverse
// Linv (lower) into linv.  One wave; lane r holds row r of the block in
// registers (by symmetry also column r).  Column c: the pivot p comes from
// lane c and each lane r > c updates its entries s > c by
// A[r][s] -= (A[r][c] / p) A[s][c], with column c read back from LDS as
// broadcasts one step ahead; then column c is scaled by 1 / sqrt(p) (one
// reciprocal square root; L[c][c] = p / sqrt(p)).  L then
// goes to LDS once (col[c][i] = L[i][c]) and Linv is built one column per
// lane by a column sweep over L: y[j] /= L[j][j], then y[i] -= L[i][j] y[j]
// for i > j, with L's column j read as 16-byte broadcasts (all lanes read one
// address).  A pivot below 1e-6 of its diagonal entry before the
// factorisation sets EINVAL: the Gram matrix plus ridge is not positive
// definite in fp32 (e.g. a zero ridge with fewer rows than dimensions).
// Run by the first wave of a workgroup (lane r = threadIdx.x); col is 16 KiB
// of 16-byte aligned LDS.
__device__ __forceinline__ void chol_diag_wave(float *G, int k, const float *dg, float *linv, int32_t *status,
                                               float (*col)[kNB]) {
  float *blk = G + (size_t)(k * kNB) * kEmb + k * kNB;
  const int r = threadIdx.x;
  float x[kNB];
#pragma unroll
  for (int q = 0; q < kNB / 4; ++q) {
    const float4 v = *reinterpret_cast<const float4 *>(blk + (size_t)r * kEmb + 4 * q);
    x[4 * q] = v.x;
    x[4 * q + 1] = v.y;
    x[4 * q + 2] = v.z;
    x[4 * q + 3] = v.w;
  }
  const float dgr = dg[k * kNB + r];
  bool bad = false;
  float dinv = 0.f;  // lane r: 1 / L[r][r]
  auto bcast = [](float v, int lane) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane)); };
  // column c of the partly factorised block goes through LDS (col[c][s] =
  // A[s][c], written by lane s) and comes back as 16-byte broadcasts; a
  // wave's LDS accesses complete in order, so a read after a write sees it.
  // Column c + 1 is updated and written first in step c and its reads are
  // issued before the rest of step c's updates, which hide their latency.
  float cv[kNB], nv[kNB];
  // pieces from q0 on (the entries before are not needed)
#define DCKV_READ_COL(c, v, q0)                                                      \
  _Pragma("unroll") for (int q = (q0); q < kNB / 4; ++q) {                          \
    const float4 t = *reinterpret_cast<const float4 *>(&col[(c)][4 * q]);            \
    v[4 * q] = t.x;                                                                  \
    v[4 * q + 1] = t.y;                                                              \
    v[4 * q + 2] = t.z;                                                              \
    v[4 * q + 3] = t.w;                                                              \
  }
  // step c with column c in cur; column c + 1 is read into nxt.  Steps go in
  // pairs so that the two buffers swap roles without copies.
#define DCKV_FACTOR_STEP(c, cur, nxt)                                               \
  {                                                                                \
    const float piv = bcast(x[(c)], (c));                                          \
    const float dgc = bcast(dgr, (c));                                             \
    bad = bad || !(piv > 1e-6f * dgc) || !isfinite(piv);                           \
    const float pc = fmaxf(piv, 1e-30f);                                           \
    const float rd = __builtin_amdgcn_rsqf(pc);                                    \
    const float l2 = r > (c) ? x[(c)] * (rd * rd) : 0.f;                           \
    if ((c) + 1 < kNB) {                                                           \
      x[(c) + 1] = fmaf(-l2, cur[(c) + 1], x[(c) + 1]);                            \
      col[(c) + 1][r] = x[(c) + 1];                                                \
      DCKV_READ_COL((c) + 1, nxt, ((c) + 2) / 4)                                   \
    }                                                                              \
    __builtin_amdgcn_sched_barrier(0);                                             \
    _Pragma("unroll") for (int s2 = (c) + 2; s2 < kNB; ++s2) x[s2] = fmaf(-l2, cur[s2], x[s2]); \
    if (r == (c)) dinv = rd;                                                       \
    x[(c)] = r == (c) ? pc * rd : (r > (c) ? x[(c)] * rd : 0.f);                   \
  }
  // A[r][s] -= (A[r][c] / p) A[s][c] for s > c; lanes at or above c leave
  // their row alone; rows above c hold upper-triangle values: set to 0,
  // zeroed in the output
  col[0][r] = x[0];
  DCKV_READ_COL(0, cv, 0)
#pragma unroll
  for (int c = 0; c < kNB; c += 2) {
    DCKV_FACTOR_STEP(c, cv, nv)
    DCKV_FACTOR_STEP(c + 1, nv, cv)
  }
#undef DCKV_FACTOR_STEP
#pragma unroll
  for (int q = 0; q < kNB / 4; ++q) {
    const float4 v = {x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]};
    *reinterpret_cast<float4 *>(blk + (size_t)r * kEmb + 4 * q) = v;
  }
  // L to LDS, transposed: col[c][r] = L[r][c] (0 above the diagonal)
#pragma unroll
  for (int c = 0; c < kNB; ++c) col[c][r] = c == r ? 0.f : x[c];
  wave_lds_sync();
  // Linv column r: L y = e_r (entries above r stay 0).  Column j of L (row j
  // of col) is read by all lanes at once, in 16-byte pieces, one column ahead
  // of its use, so the reads never wait on the sweep.
  float y[kNB];
#pragma unroll
  for (int i = 0; i < kNB; ++i) y[i] = i == r ? 1.f : 0.f;
#define DCKV_SWEEP_STEP(j, cur, nxt)                                               \
  {                                                                                \
    if ((j) + 1 < kNB) DCKV_READ_COL((j) + 1, nxt, ((j) + 2) / 4)                  \
    __builtin_amdgcn_sched_barrier(0);                                             \
    y[(j)] *= bcast(dinv, (j));                                                    \
    _Pragma("unroll") for (int i = (j) + 1; i < kNB; ++i) y[i] = fmaf(-cur[i], y[(j)], y[i]); \
  }
  DCKV_READ_COL(0, cv, 0)
#pragma unroll
  for (int j = 0; j < kNB; j += 2) {
    DCKV_SWEEP_STEP(j, cv, nv)
    DCKV_SWEEP_STEP(j + 1, nv, cv)
  }
#undef DCKV_SWEEP_STEP
#undef DCKV_READ_COL
  float *lv = linv + (size_t)k * kNB * kNB;
#pragma unroll
  for (int i = 0; i < kNB; ++i) lv[i * kNB + r] = y[i];
  if (r == 0 && bad) atomicCAS(status, 0, DCKV_EINVAL);
}

// The first diagonal block (the later ones are factorised inside the trailing
// update that finishes them).
__global__ __launch_bounds__(64) void k_chol_diag(float *G, int k, const float *dg, float *linv, int32_t *status) {
  __shared__ __attribute__((aligned(16))) float col[kNB][kNB];
  chol_diag_wave(G, k, dg, linv, status, col);
}

// 64 x 64 tile products on 256 threads.  Operands are staged in LDS as
// P[t][r] = op(A)(r, t) and Q[t][s] = op(B)(t, s) (rows padded to 65 floats:
// conflict-free transposed writes); thread (r0, s0) = (tid / 16 * 4,
// tid % 16 * 4) accumulates the 4 x 4 block at rows r0.., columns s0..
typedef float TileLds[kNB][kNB + 1];

// s[p][q] = M[p][q] (kDirect) or s[q][p] = M[p][q], M row-major with leading
// dimension ld (a multiple of 4, 16-byte aligned rows); 16-byte reads, four
// per thread, coalesced along q.  A wave's 64 reads cover 4 rows x 16 quads,
// so with rows padded to 65 floats the scalar LDS writes (p + q + e, mod 64)
// fall in distinct banks either way.
template <bool kDirect>
__device__ __forceinline__ void stage(TileLds &s, const float *M, int ld) {
  float4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int f = threadIdx.x + 256 * u, p = f >> 4, q = (f & 15) * 4;
    v[u] = *reinterpret_cast<const float4 *>(M + (size_t)p * ld + q);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int f = threadIdx.x + 256 * u, p = f >> 4, q = (f & 15) * 4;
    const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (kDirect) s[p][q + i] = e[i]; else s[q + i][p] = e[i];
    }
  }
}

__device__ __forceinline__ void tile_mac(const TileLds &P, const TileLds &Q, float (&acc)[4][4]) {
  const int r0 = (threadIdx.x >> 4) * 4, s0 = (threadIdx.x & 15) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
#pragma unroll 8
  for (int t = 0; t < kNB; ++t) {
    float av[4], bv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      av[i] = P[t][r0 + i];
      bv[i] = Q[t][s0 + i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
  }
}

// this thread's 4 x 4 block of a row-major tile, as four 16-byte rows
__device__ __forceinline__ void load_block(const float *C, int ldc, float (&v)[4][4]) {
  const int r0 = (threadIdx.x >> 4) * 4, s0 = (threadIdx.x & 15) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 w = *reinterpret_cast<const float4 *>(C + (size_t)(r0 + i) * ldc + s0);
    v[i][0] = w.x;
    v[i][1] = w.y;
    v[i][2] = w.z;
    v[i][3] = w.w;
  }
}

__device__ __forceinline__ void store_block(float *C, int ldc, const float (&v)[4][4]) {
  const int r0 = (threadIdx.x >> 4) * 4, s0 = (threadIdx.x & 15) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<float4 *>(C + (size_t)(r0 + i) * ldc + s0) = make_float4(v[i][0], v[i][1], v[i][2], v[i][3]);
}

// C = op(A) op(B) (kAcc false) or C -= op(A) op(B), with op(A)(r, t) = A[r][t]
// (A[t][r] when kTA) and op(B)(t, s) = B[t][s] (B[s][t] when kTB).  Both
// operands are in LDS before C is written, so C may be one of them.  The
// result stays in v for a caller that applies a second product.
template <bool kTA, bool kTB, bool kAcc>
__device__ __forceinline__ void tile_op(TileLds &P, TileLds &Q, float *C, int ldc, const float *A, int lda,
                                        const float *B, int ldb, float (&v)[4][4]) {
  if (kAcc) load_block(C, ldc, v);  // in flight while the operands are staged
  stage<kTA>(P, A, lda);
  stage<!kTB>(Q, B, ldb);
  __syncthreads();
  float acc[4][4];
  tile_mac(P, Q, acc);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) v[i][j] = kAcc ? v[i][j] - acc[i][j] : acc[i][j];
  store_block(C, ldc, v);
}

// After diagonal block k (m = block rows below it): workgroups x < m form the
// panel L_ik = G_ik Linv_kk^T (i = k + 1 + x); the next 32 take the forward
// substitution's diagonal step on the right-hand sides X [kEmb][kC]:
// X_k = Linv_kk X_k, one 64-column block each.
__global__ __launch_bounds__(256) void k_chol_panel_fwd(float *G, float *X, const float *linv, int k, int m) {
  __shared__ TileLds P, Q;
  float v[4][4];
  const float *lk = linv + (size_t)k * kNB * kNB;
  if ((int)blockIdx.x < m) {
    float *gik = G + (size_t)((k + 1 + blockIdx.x) * kNB) * kEmb + k * kNB;
    tile_op<false, true, false>(P, Q, gik, kEmb, gik, kEmb, lk, kNB, v);
  } else {
    float *xk = X + (size_t)(k * kNB) * kC + (blockIdx.x - m) * kNB;
    tile_op<false, false, false>(P, Q, xk, kC, lk, kNB, xk, kC, v);
  }
}

// The trailing update after panel k, with the forward substitution's update:
// the first m (m + 1) / 2 workgroups take G_ij -= L_ik L_jk^T over the lower
// triangle k < j <= i; the next 32 m take X_i -= L_ik X_k (i > k, one
// 64-column block each).  Workgroup 0 updates diagonal block k + 1, which is
// then final, and its first wave factorises it (chol_diag_wave) while the
// other workgroups finish the update: the factorisation of one block no
// longer runs alone on the chip between two launches.  Two workgroups per CU
// leave the factorisation its registers.
__global__ __launch_bounds__(256, 2) void k_chol_update_fwd(float *G, float *X, int k, int m, const float *dg,
                                                            float *linv, int32_t *status) {
  __shared__ __attribute__((aligned(16))) TileLds P, Q;
  float v[4][4];
  const int t = blockIdx.x, ntri = m * (m + 1) / 2;
  if (t < ntri) {
    int ii = (int)((sqrtf(8.f * (float)t + 1.f) - 1.f) * 0.5f);
    while ((ii + 1) * (ii + 2) / 2 <= t) ++ii;
    while (ii * (ii + 1) / 2 > t) --ii;
    const int i = k + 1 + ii, j = k + 1 + (t - ii * (ii + 1) / 2);
    tile_op<false, true, true>(P, Q, G + (size_t)(i * kNB) * kEmb + j * kNB, kEmb, G + (size_t)(i * kNB) * kEmb + k * kNB,
                               kEmb, G + (size_t)(j * kNB) * kEmb + k * kNB, kEmb, v);
    if (t == 0) {
      // the block's stores are visible to the workgroup and P is free
      __syncthreads();
      static_assert(sizeof(TileLds) >= kNB * kNB * sizeof(float), "column buffer inside P");
      if (threadIdx.x < kNB) chol_diag_wave(G, k + 1, dg, linv, status, reinterpret_cast<float (*)[kNB]>(&P[0][0]));
    }
  } else {
    const int u = t - ntri, i = k + 1 + u / (kC / kNB), c0 = (u % (kC / kNB)) * kNB;
    tile_op<false, false, true>(P, Q, X + (size_t)(i * kNB) * kC + c0, kC, G + (size_t)(i * kNB) * kEmb + k * kNB, kEmb,
                                X + (size_t)(k * kNB) * kC + c0, kC, v);
  }
}

// Backward substitution L^T X = Z, last block row: X_k = Linv_kk^T X_k.
__global__ __launch_bounds__(256) void k_bwd_diag(float *X, const float *linv, int k) {
  __shared__ TileLds P, Q;
  float v[4][4];
  float *xk = X + (size_t)(k * kNB) * kC + blockIdx.x * kNB;
  tile_op<true, false, false>(P, Q, xk, kC, linv + (size_t)k * kNB * kNB, kNB, xk, kC, v);
}

// Backward step k (X_k final): X_i -= L_ki^T X_k for i < k, blockIdx =
// (i, 64-column block); the workgroups of row i = k - 1 then finish it,
// X_{k-1} = Linv^T X_{k-1}, from the registers they hold.
__global__ __launch_bounds__(256) void k_bwd_step(float *X, const float *G, const float *linv, int k) {
  __shared__ TileLds P, Q;
  float v[4][4];
  const int i = blockIdx.x, c0 = blockIdx.y * kNB;
  float *xi = X + (size_t)(i * kNB) * kC + c0;
  tile_op<true, false, true>(P, Q, xi, kC, G + (size_t)(k * kNB) * kEmb + i * kNB, kEmb, X + (size_t)(k * kNB) * kC + c0,
                             kC, v);
  if (i != k - 1) return;
  __syncthreads();  // every thread is done with P and Q
  const int r0 = (threadIdx.x >> 4) * 4, s0 = (threadIdx.x & 15) * 4;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) Q[r0 + a][s0 + b] = v[a][b];
  stage<true>(P, linv + (size_t)i * kNB * kNB, kNB);  // P[t][r] = Linv[t][r] = op(A)(r, t) of Linv^T
  __syncthreads();
  float acc[4][4];
  tile_mac(P, Q, acc);
  store_block(xi, kC, acc);
}
// H[c][e] = Ht[e][c] (fp32 out), Hb = bf16(H)
__global__ void k_fit_h_out(const float *Ht, float *H, uint16_t *Hb, uint16_t *Hb2) {
  __shared__ float t[64][65];
  const int c0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) t[r][tx] = Ht[(size_t)(e0 + r) * kC + c0 + tx];
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const float h = t[tx][r];
    const size_t o = (size_t)(c0 + r) * kEmb + e0 + tx;
    if (H) H[o] = h;
    Hb[o] = f2bf(h);
    if (Hb2) Hb2[o] = f2bf(h);
  }
}

// Per-component sums over one chunk of rows (blockIdx.y), one thread per
// component (consecutive components: coalesced rows).  Phase 0: sum r s and
// sum s^2 over the chunk's odd rows; phase 1: sum |y - mu| over all its rows,
// with the fitted a.  The partial sums are fp64; the chunks are added in a
// fixed order by k_fit_ab_reduce.
template <int kPhase>
__global__ void k_fit_ab_part(const float *Y, const float *M, int64_t n, int64_t rows_per, const float *a,
                              double *part) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t j0 = (int64_t)blockIdx.y * rows_per, j1 = min<int64_t>(n, j0 + rows_per);
  auto y = [&](int64_t j) { return j >= 0 && j < n ? (double)Y[(size_t)j * kC + c] : 0.0; };
  if (kPhase == 0) {
    double num = 0.0, den = 0.0;
    for (int64_t j = j0 | 1; j < j1; j += 2) {
      const double sn = y(j - 1) + y(j + 1);
      const double r = y(j) - (double)M[(size_t)j * kC + c];
      num += r * sn;
      den += sn * sn;
    }
    part[((size_t)blockIdx.y * 2) * kC + c] = num;
    part[((size_t)blockIdx.y * 2 + 1) * kC + c] = den;
  } else {
    const double ac = a[c];
    double sum = 0.0;
    for (int64_t j = j0; j < j1; ++j) {
      double mu = M[(size_t)j * kC + c];
      if (j & 1) mu += ac * (y(j - 1) + y(j + 1));
      sum += fabs(y(j) - mu);
    }
    part[(size_t)blockIdx.y * kC + c] = sum;
  }
}

// The chunk sums of 64 components per workgroup: wave w adds the chunks
// i = w, w + 4, ... of its lane's component in order, then the four wave
// sums are added in wave order (a fixed order, so the result does not vary
// between runs).
template <int kPhase>
__global__ __launch_bounds__(256) void k_fit_ab_reduce(const double *part, int chunks, int64_t n, float *out) {
  __shared__ double acc[2][4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  double s0 = 0.0, s1 = 0.0;
#pragma unroll 4
  for (int i = w; i < chunks; i += 4) {
    if (kPhase == 0) {
      s0 += part[((size_t)i * 2) * kC + c];
      s1 += part[((size_t)i * 2 + 1) * kC + c];
    } else {
      s0 += part[(size_t)i * kC + c];
    }
  }
  acc[0][w][lane] = s0;
  acc[1][w][lane] = s1;
  __syncthreads();
  if (w != 0) return;
  double num = 0.0, den = 0.0;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    num += acc[0][v][lane];
    den += acc[1][v][lane];
  }
  if (kPhase == 0)
    out[c] = den > 0.0 ? (float)(num / den) : 0.f;
  else
    out[c] = (float)(num / (double)n);
}

}  // namespace

void launch_clear_status(int32_t *status, hipStream_t s) {
  hipLaunchKernelGGL(k_fit_clear_status, dim3(1), dim3(1), 0, s, status);
}

void launch_gather_t(const uint16_t *E, const int32_t *tok, int64_t n, int64_t n_pad, int vocab, uint16_t *Et,
                     int32_t *tokc, int32_t *status, hipStream_t s) {
  hipLaunchKernelGGL(k_fit_gather_t, dim3((unsigned)(n_pad / 64), kEmb / 64), dim3(256), 0, s, E, tok, n, n_pad,
                     vocab, Et, tokc, status);
}

void launch_split_t(const float *Y, int64_t n, int64_t n_pad, uint16_t *hi, uint16_t *lo, hipStream_t s) {
  hipLaunchKernelGGL(k_fit_split_t, dim3((unsigned)(n_pad / 64), kC / 64), dim3(256), 0, s, Y, n, n_pad, hi, lo);
}

FitLayout fit_layout(int64_t n) {
  FitLayout l;
  l.n_pad = (n + 63) / 64 * 64;
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t o = off;
    off = (off + bytes + 255) / 256 * 256;
    return o;
  };
  l.Y = take((uint64_t)n * kC * 4);
  l.M = take((uint64_t)n * kC * 4);
  l.Yhi = take((uint64_t)kC * l.n_pad * 2);
  l.Ylo = take((uint64_t)kC * l.n_pad * 2);
  l.Et = take((uint64_t)kEmb * l.n_pad * 2);
  l.G = take((uint64_t)kEmb * kEmb * 4);
  l.R = take((uint64_t)kEmb * kC * 4);
  l.Hb = take((uint64_t)kC * kEmb * 2);
  l.tokc = take((uint64_t)n * 4);
  l.part = take((uint64_t)kFitChunks * 2 * kC * 8);
  l.dg = take((uint64_t)kEmb * 4);
  l.linv = take((uint64_t)kNBlk * kNB * kNB * 4);
  l.total = off;
  return l;
}

void fit_sequence(const FitArgs &a) {
  const FitLayout &l = a.l;
  uint8_t *ws = a.ws;
  float *Y = reinterpret_cast<float *>(ws + l.Y), *M = reinterpret_cast<float *>(ws + l.M);
  uint16_t *Yhi = reinterpret_cast<uint16_t *>(ws + l.Yhi), *Ylo = reinterpret_cast<uint16_t *>(ws + l.Ylo);
  uint16_t *Et = reinterpret_cast<uint16_t *>(ws + l.Et), *Hb = reinterpret_cast<uint16_t *>(ws + l.Hb);
  float *G = reinterpret_cast<float *>(ws + l.G), *R = reinterpret_cast<float *>(ws + l.R);
  const int64_t n = a.n, np = l.n_pad;
  const hipStream_t s = a.s;
  hipLaunchKernelGGL(k_fit_clear_status, dim3(1), dim3(1), 0, s, a.status);
  int32_t *tokc = reinterpret_cast<int32_t *>(ws + l.tokc);
  double *part = reinterpret_cast<double *>(ws + l.part);
  hipLaunchKernelGGL(k_fit_gather_t, dim3((unsigned)(np / 64), kEmb / 64), dim3(256), 0, s, a.E, a.tok, n, np,
                     a.vocab, Et, tokc, a.status);
  GemmF32Args g{};
  // Y = X A^T
  g.a0 = g.a1 = a.rows;
  g.lda0 = g.lda1 = kD * 2;
  g.b0 = g.b1 = a.A;
  g.ldb0 = g.ldb1 = kD * 2;
  g.KT = g.split = kD / kBK;
  g.arow = nullptr;
  g.M = (int)n;
  g.N = kC;
  g.c = Y;
  g.ldc = kC;
  launch_gemm_f32(g, s);
  hipLaunchKernelGGL(k_fit_split_t, dim3((unsigned)(np / 64), kC / 64), dim3(256), 0, s, Y, n, np, Yhi, Ylo);
  // G = Et Et^T and R = Et [Yhi | Ylo]^T (= E^T Y with 16 mantissa bits of Y):
  // independent, 64 tiles each, so one launch
  g.a0 = g.a1 = Et;
  g.lda0 = g.lda1 = (uint32_t)(np * 2);
  g.b0 = g.b1 = Et;
  g.ldb0 = g.ldb1 = (uint32_t)(np * 2);
  g.KT = g.split = (int)(np / kBK);
  g.M = kEmb;
  g.N = kEmb;
  g.c = G;
  g.ldc = kEmb;
  GemmF32Args gr = g;
  gr.b0 = Yhi;
  gr.b1 = Ylo;
  gr.KT = (int)(2 * np / kBK);
  gr.split = (int)(np / kBK);
  gr.N = kC;
  gr.c = R;
  gr.ldc = kC;
  launch_gemm_f32_pair(g, gr, s);
  g = gr;
  float *dg = reinterpret_cast<float *>(ws + l.dg);
  float *linv = reinterpret_cast<float *>(ws + l.linv);
  hipLaunchKernelGGL(k_fit_add_diag, dim3(kEmb / 256), dim3(256), 0, s, G, a.ridge * (float)n, dg);
  // G = L L^T by blocks, with the forward substitution L Z = R riding along:
  // the first diagonal block, then per block k one panel launch (plus Z_k)
  // and one trailing-update launch (plus R_i -= L_ik Z_k) that also
  // factorises diagonal block k + 1
  hipLaunchKernelGGL(k_chol_diag, dim3(1), dim3(64), 0, s, G, 0, dg, linv, a.status);
  for (int k = 0; k < kNBlk; ++k) {
    const int m = kNBlk - k - 1;
    hipLaunchKernelGGL(k_chol_panel_fwd, dim3(m + kC / kNB), dim3(256), 0, s, G, R, linv, k, m);
    if (m > 0)
      hipLaunchKernelGGL(k_chol_update_fwd, dim3(m * (m + 1) / 2 + m * (kC / kNB)), dim3(256), 0, s, G, R, k, m,
                         (const float *)dg, linv, a.status);
  }
  // L^T H^T = Z: one launch per block row
  hipLaunchKernelGGL(k_bwd_diag, dim3(kC / kNB), dim3(256), 0, s, R, linv, kNBlk - 1);
  for (int k = kNBlk - 1; k > 0; --k) hipLaunchKernelGGL(k_bwd_step, dim3(k, kC / kNB), dim3(256), 0, s, R, G, linv, k);
  hipLaunchKernelGGL(k_fit_h_out, dim3(kC / 64, kEmb / 64), dim3(256), 0, s, R, a.H_out, Hb, a.Hb_out);
  // M = E[tok] bf16(H)^T
  g.a0 = g.a1 = a.E;
  g.lda0 = g.lda1 = kEmb * 2;
  g.b0 = g.b1 = Hb;
  g.ldb0 = g.ldb1 = kEmb * 2;
  g.KT = g.split = kEmb / kBK;
  g.arow = tokc;
  g.M = (int)n;
  g.N = kC;
  g.c = M;
  g.ldc = kC;
  launch_gemm_f32(g, s);
  // chunks of an even number of rows, so that odd rows keep their parity
  const int64_t per = ((n + kFitChunks - 1) / kFitChunks + 1) / 2 * 2;
  const int chunks = (int)((n + per - 1) / per);
  hipLaunchKernelGGL(k_fit_ab_part<0>, dim3(kC / 256, chunks), dim3(256), 0, s, Y, M, n, per, a.a_out, part);
  hipLaunchKernelGGL(k_fit_ab_reduce<0>, dim3(kC / 64), dim3(256), 0, s, part, chunks, n, a.a_out);
  hipLaunchKernelGGL(k_fit_ab_part<1>, dim3(kC / 256, chunks), dim3(256), 0, s, Y, M, n, per, a.a_out, part);
  hipLaunchKernelGGL(k_fit_ab_reduce<1>, dim3(kC / 64), dim3(256), 0, s, part, chunks, n, a.b_out);
}

}  // namespace dckv
