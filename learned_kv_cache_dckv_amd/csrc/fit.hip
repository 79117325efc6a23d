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

// Unblocked Cholesky of diagonal block k (lower, in place; the block's upper
// triangle is zeroed, so later kernels read it as L_kk), then its inverse
// Linv (lower) into linv.  One wave: lane r holds row r in registers; column
// c's entries of the other rows come by readlane.  A pivot below 1e-6 of its
// diagonal entry before the factorisation sets EINVAL: the Gram matrix plus
// ridge is not positive definite in fp32 (e.g. a zero ridge with fewer rows
// than dimensions).
__global__ __launch_bounds__(64) void k_chol_diag(float *G, int k, const float *dg, float *linv, int32_t *status) {
  __shared__ float l[kNB][kNB + 1];
  float *blk = G + (size_t)(k * kNB) * kEmb + k * kNB;
  const int r = threadIdx.x;
  float x[kNB];
#pragma unroll
  for (int s = 0; s < kNB; ++s) x[s] = blk[(size_t)r * kEmb + s];
  bool bad = false;
#pragma unroll
  for (int c = 0; c < kNB; ++c) {
    const float piv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x[c]), c));
    bad = bad || !(piv > 1e-6f * dg[k * kNB + c]) || !isfinite(piv);
    const float d = sqrtf(fmaxf(piv, 1e-30f));
    x[c] = r == c ? d : x[c] / d;  // rows above c hold upper-triangle values: discarded
    // x[s] -= L[r][c] L[s][c] for s > c (L[s][c] is lane s's x[c])
#pragma unroll
    for (int s = c + 1; s < kNB; ++s)
      x[s] -= x[c] * __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x[c]), s));
  }
#pragma unroll
  for (int s = 0; s < kNB; ++s) {
    const float v = s <= r ? x[s] : 0.f;
    l[r][s] = v;
    blk[(size_t)r * kEmb + s] = v;
  }
  __syncthreads();
  // Linv column r: L y = e_r by forward substitution (rows above r are 0)
  float y[kNB];
#pragma unroll
  for (int i = 0; i < kNB; ++i) {
    float v = i == r ? 1.f : 0.f;
#pragma unroll
    for (int j = 0; j < i; ++j) v -= l[i][j] * y[j];
    y[i] = i < r ? 0.f : v / l[i][i];
  }
  float *lv = linv + (size_t)k * kNB * kNB;
#pragma unroll
  for (int i = 0; i < kNB; ++i) lv[i * kNB + r] = y[i];
  if (r == 0 && bad) atomicCAS(status, 0, DCKV_EINVAL);
}

// One 64 x 64 tile: C = op(A) op(B) (kAcc false) or C -= op(A) op(B), with
// op(A)(r, t) = A[r][t] (A[t][r] when kTA) and op(B)(t, s) = B[t][s] (B[s][t]
// when kTB); row-major with the given leading dimensions.  Both operands are
// read into LDS before C is written, so C may be one of them.
template <bool kTA, bool kTB, bool kAcc>
__device__ __forceinline__ void tile_op(float *C, int ldc, const float *A, int lda, const float *B, int ldb) {
  __shared__ float sa[kNB][kNB + 1];  // sa[t][r]
  __shared__ float sb[kNB][kNB + 1];  // sb[t][s]
  const int tid = threadIdx.x;
  for (int i = tid; i < kNB * kNB; i += 256) {
    const int p = i / kNB, q = i % kNB;  // row p, column q of the stored matrix (coalesced in q)
    const float av = A[(size_t)p * lda + q];
    if (kTA) sa[p][q] = av; else sa[q][p] = av;
    const float bv = B[(size_t)p * ldb + q];
    if (kTB) sb[q][p] = bv; else sb[p][q] = bv;
  }
  __syncthreads();
  const int r0 = (tid >> 4) * 4, s0 = (tid & 15) * 4;
  float acc[4][4] = {};
#pragma unroll 8
  for (int t = 0; t < kNB; ++t) {
    float av[4], bv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      av[i] = sa[t][r0 + i];
      bv[i] = sb[t][s0 + i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float &c = C[(size_t)(r0 + i) * ldc + s0 + j];
      c = kAcc ? c - acc[i][j] : acc[i][j];
    }
}

// Panel: L_ik = G_ik Linv_kk^T for the block rows i = k + 1 + blockIdx.x.
__global__ __launch_bounds__(256) void k_chol_panel(float *G, const float *linv, int k) {
  float *gik = G + (size_t)((k + 1 + blockIdx.x) * kNB) * kEmb + k * kNB;
  tile_op<false, true, false>(gik, kEmb, gik, kEmb, linv + (size_t)k * kNB * kNB, kNB);
}

// Cholesky trailing update after block k: G_ij -= L_ik L_jk^T for
// k < j <= i; blockIdx = (i - k - 1, j - k - 1).
__global__ __launch_bounds__(256) void k_chol_update(float *G, int k) {
  const int i = k + 1 + blockIdx.x, j = k + 1 + blockIdx.y;
  if (j > i) return;
  tile_op<false, true, true>(G + (size_t)(i * kNB) * kEmb + j * kNB, kEmb, G + (size_t)(i * kNB) * kEmb + k * kNB,
                           kEmb, G + (size_t)(j * kNB) * kEmb + k * kNB, kEmb);
}

// Right-hand sides X [kEmb][kC] (row-major): block row k times Linv_kk
// (forward, X_k = L_kk^-1 X_k) or Linv_kk^T (backward, X_k = L_kk^-T X_k),
// one 64-column block per workgroup.
template <bool kFwd>
__global__ __launch_bounds__(256) void k_solve_diag(float *X, const float *linv, int k) {
  float *xk = X + (size_t)(k * kNB) * kC + blockIdx.x * kNB;
  tile_op<!kFwd, false, false>(xk, kC, linv + (size_t)k * kNB * kNB, kNB, xk, kC);
}

// After block row k is solved: forward, X_i -= L_ik X_k for i > k; backward,
// X_i -= L_ki^T X_k for i < k.  blockIdx = (block row index among those,
// 64-column block of the right-hand sides).
template <bool kFwd>
__global__ __launch_bounds__(256) void k_solve_update(float *X, const float *G, int k) {
  const int i = kFwd ? k + 1 + blockIdx.x : blockIdx.x;
  const int c0 = blockIdx.y * kNB;
  float *Ci = X + (size_t)(i * kNB) * kC + c0;
  const float *Xk = X + (size_t)(k * kNB) * kC + c0;
  if (kFwd)
    tile_op<false, false, true>(Ci, kC, G + (size_t)(i * kNB) * kEmb + k * kNB, kEmb, Xk, kC);
  else
    tile_op<true, false, true>(Ci, kC, G + (size_t)(k * kNB) * kEmb + i * kNB, kEmb, Xk, kC);
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

template <int kPhase>
__global__ void k_fit_ab_reduce(const double *part, int chunks, int64_t n, float *out) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (kPhase == 0) {
    double num = 0.0, den = 0.0;
    for (int i = 0; i < chunks; ++i) {
      num += part[((size_t)i * 2) * kC + c];
      den += part[((size_t)i * 2 + 1) * kC + c];
    }
    out[c] = den > 0.0 ? (float)(num / den) : 0.f;
  } else {
    double sum = 0.0;
    for (int i = 0; i < chunks; ++i) sum += part[(size_t)i * kC + c];
    out[c] = (float)(sum / (double)n);
  }
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
  for (int k = 0; k < kNBlk; ++k) {
    hipLaunchKernelGGL(k_chol_diag, dim3(1), dim3(64), 0, s, G, k, dg, linv, a.status);
    const int m = kNBlk - k - 1;
    if (m > 0) {
      hipLaunchKernelGGL(k_chol_panel, dim3(m), dim3(256), 0, s, G, linv, k);
      hipLaunchKernelGGL(k_chol_update, dim3(m, m), dim3(256), 0, s, G, k);
    }
  }
  for (int k = 0; k < kNBlk; ++k) {  // L Z = R
    hipLaunchKernelGGL(k_solve_diag<true>, dim3(kC / kNB), dim3(256), 0, s, R, linv, k);
    if (k + 1 < kNBlk)
      hipLaunchKernelGGL(k_solve_update<true>, dim3(kNBlk - k - 1, kC / kNB), dim3(256), 0, s, R, G, k);
  }
  for (int k = kNBlk - 1; k >= 0; --k) {  // L^T H^T = Z
    hipLaunchKernelGGL(k_solve_diag<false>, dim3(kC / kNB), dim3(256), 0, s, R, linv, k);
    if (k > 0) hipLaunchKernelGGL(k_solve_update<false>, dim3(k, kC / kNB), dim3(256), 0, s, R, G, k);
  }
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
  hipLaunchKernelGGL(k_fit_ab_reduce<0>, dim3(kC / 256), dim3(256), 0, s, part, chunks, n, a.a_out);
  hipLaunchKernelGGL(k_fit_ab_part<1>, dim3(kC / 256, chunks), dim3(256), 0, s, Y, M, n, per, a.a_out, part);
  hipLaunchKernelGGL(k_fit_ab_reduce<1>, dim3(kC / 256), dim3(256), 0, s, part, chunks, n, a.b_out);
}

}  // namespace dckv
