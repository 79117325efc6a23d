// The rate term of codec training and its gradients (DCKV digest page, "How
// it works", Training bullet: the rate is the code length of coefficients
// perturbed by uniform noise; the reconstruction uses the quantised values,
// and its gradient bypasses the rounding).
//
// For coded row j and active component c, with step D, Laplace scale b,
// s = b / D, neighbour weight a and embedding mean m:
//   even j: mu = m;  odd j: mu = m + a (yhat_{j-1} + yhat_{j+1}), yhat_N = 0
//   q = rint(fp32(y - mu) / D),  yhat = mu + q D     (the codec's two passes)
//   t = (y - mu) / D + u,        u the caller's noise in steps
//   bits = -log2(F_s(t + 1/2) - F_s(t - 1/2)),  F_s the zero-mean Laplace CDF
// and, with beta = d bits / dt and gamma = d bits / ds,
//   dR/dm_j = -beta_j / D
//   dR/dy_j = beta_j / D, plus a (dR/dm_{j-1} + dR/dm_{j+1}) on even rows
//             (their reconstruction is in the odd neighbours' means)
//   dR/da   = sum over odd j of dR/dm_j (yhat_{j-1} + yhat_{j+1})
//   dR/db   = sum over j of gamma_j / D.
// Dropped components: bits 0, yhat = mu, no gradient.  Through y = A x and
// m = H e the weight gradients are dR/dA = sum_j dR/dy_j x_j^T and
// dR/dH = sum_j dR/dm_j e_j^T.
//
// Work split: the coefficients y = A x come from the fp32-output GEMM (split
// over k into two partial sets when its tiles alone would not fill the chip);
// one thread per component codes a chunk of rows held in registers, so the
// neighbour terms are register reads (the two rows before the chunk and the
// one after it are recomputed).  Per-token bits are column-block sums written
// as partials and added in a fixed order; the per-component sums are fp64
// within a chunk, stored per chunk and added in fp64 by two reduction kernels,
// the second of which also sets the status.  The weight gradients are two
// MFMA products over the token dimension in one launch.
#include "dckv_internal.h"

namespace dckv {
namespace {

constexpr int kRateRows = 16;    // rows per chunk (even)
constexpr int kRateCols = 256;   // components per workgroup
constexpr int kRateParts = kC / kRateCols;  // column-block partials per row

struct RateP {
  const float *Y;        // [ksplit][N][C] partial coefficients
  const float *mtab;     // [vocab][C] embedding means, plan column order
  const int32_t *tok;    // [T]
  const float *noise;    // [N][C]
  const float *step, *nbr, *scale;
  const int32_t *rank, *colpos;
  float *yhat, *gy, *gm;  // [N][C]
  float *bits_part;       // [kRateParts][N]
  float *ga_part, *gb_part;   // [chunks][C] per-chunk sums (fp64 inside a chunk)
  int32_t *flags;             // [chunks][C / kRateCols] a bad input seen
  int64_t N, chunks;          // chunks of kRateRows rows
  int keep_head, vocab, ksplit;  // ksplit 1 or 2
};

struct Col {
  float step, a, s, inv_s_l2, k0, g0;
  bool act;
  int col;
};

struct Out {
  float yhat, beta, gamma, bits;
};

constexpr float kLog2e = 1.4426950408889634f;

// code length of the noisy residual t (in steps) and its derivatives
__device__ __forceinline__ void rate_of(float t, const Col &k, Out &o) {
  const float at = fabsf(t);
  const float sg = t > 0.f ? 1.f : (t < 0.f ? -1.f : 0.f);
  if (at >= 0.5f) {
    // one side of zero: P = (1/2) exp(-(|t| - 1/2)/s) (1 - exp(-1/s))
    const float v = at - 0.5f;
    o.bits = k.k0 + v * k.inv_s_l2;
    o.beta = sg * k.inv_s_l2;
    o.gamma = (k.g0 - v) * k.inv_s_l2 / k.s;
  } else {
    // P = 1 - (1/2) exp(-a1) - (1/2) exp(-a2), a1,2 = (1/2 -+ |t|)/s
    const float a1 = (0.5f - at) / k.s, a2 = (0.5f + at) / k.s;
    const float e1 = expm1f(-a1), e2 = expm1f(-a2);
    const float P = -0.5f * (e1 + e2);
    const float w = 1.f / (2.f * k.s * P) * kLog2e;
    o.bits = -log2f(P);
    o.beta = sg * (e1 - e2) * w;
    o.gamma = ((1.f + e1) * a1 + (1.f + e2) * a2) * w;
  }
}

__device__ __forceinline__ float wave_sum16(float v) {
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// reconstruction and rate of one row given its conditional mean
__device__ __forceinline__ Out code_row(float y, float u, float mu, const Col &k, bool &bad) {
  Out o;
  if (!k.act) {
    o.yhat = mu;
    o.beta = o.gamma = o.bits = 0.f;
    return o;
  }
  const float d = y - mu;
  if (!isfinite(d)) bad = true;
  const float rr = __fdiv_rn(d, k.step);
  const float q = fminf(fmaxf(rintf(rr), -2147483520.0f), 2147483520.0f);
  o.yhat = fmaf(q, k.step, mu);
  rate_of(rr + u, k, o);
  return o;
}

constexpr int kWin = kRateRows + 3;  // window rows j0 - 2 .. j0 + kRateRows

// Workgroup (column block, chunk of kRateRows rows from j0): every load of the
// chunk's window is issued first (token ids, then coefficients, noise and
// means), the rows are coded in registers, and the per-token bits of the
// block's columns are summed through LDS.
__global__ __launch_bounds__(kRateCols) void k_rate(RateP P) {
  __shared__ float lb[kRateRows * kRateCols];
  // workgroups are dealt to the 8 XCDs in turn; give each XCD a contiguous
  // range of (chunk, column block) pairs, so that it reads whole rows and the
  // halo rows of its chunks are mostly in its own L2
  const int total = (int)gridDim.x, x = blockIdx.x & 7, kk = blockIdx.x >> 3;
  const int q8 = total >> 3, r8 = total & 7;
  const int t = x < r8 ? x * (q8 + 1) + kk : r8 * (q8 + 1) + (x - r8) * q8 + kk;
  const int cb = t % kRateParts, chunk = t / kRateParts;
  const int lt = threadIdx.x;
  const int c = cb * kRateCols + lt;
  const int64_t j0 = (int64_t)chunk * kRateRows;
  const int64_t base = j0 - 2;
  Col k;
  k.step = P.step[c];
  k.a = P.nbr[c];
  k.act = P.rank[c] >= 0;
  k.col = P.colpos[c];
  k.s = P.scale[c] / k.step;
  k.inv_s_l2 = kLog2e / k.s;
  k.k0 = 1.f - log2f(-expm1f(-1.f / k.s));
  k.g0 = 1.f / expm1f(1.f / k.s);
  const float inv_d = 1.f / k.step;
  bool bad = false;
  double ga = 0.0, gb = 0.0;
  int tk[kWin];
#pragma unroll
  for (int r = 0; r < kWin; ++r) {
    const int64_t j = base + r;
    int v = 0;
    if (j >= 0 && j < P.N) {
      v = P.tok[j + P.keep_head];
      if ((unsigned)v >= (unsigned)P.vocab) {
        bad = true;
        v = 0;
      }
    }
    tk[r] = v;
  }
  // (the second partial set is added only after every load is in flight)
  float ys[kWin], y2[kWin], us[kWin], ms[kWin];
  const bool two = P.ksplit > 1;
  const int64_t NC = P.N * kC;
#pragma unroll
  for (int r = 0; r < kWin; ++r) {
    const int64_t j = base + r;
    ys[r] = y2[r] = us[r] = ms[r] = 0.f;
    if (j >= 0 && j < P.N) {
      const int64_t o = j * kC + c;
      ys[r] = P.Y[o];
      if (two) y2[r] = P.Y[NC + o];
      us[r] = P.noise[o];
      ms[r] = P.mtab[(int64_t)tk[r] * kC + k.col];
    }
  }
#pragma unroll
  for (int r = 0; r < kWin; ++r) ys[r] += y2[r];
  // even window rows 2i (rows past N reconstruct to 0: the missing neighbour)
  Out ev[kRateRows / 2 + 2];
#pragma unroll
  for (int i = 0; i < kRateRows / 2 + 2; ++i) {
    const int64_t j = base + 2 * i;
    ev[i] = Out{0.f, 0.f, 0.f, 0.f};
    if (j >= 0 && j < P.N) ev[i] = code_row(ys[2 * i], us[2 * i], ms[2 * i], k, bad);
  }
  // odd window rows 2i + 1, with the neighbours' reconstruction in their means
  Out od[kRateRows / 2 + 1];
  float nbs[kRateRows / 2 + 1];
#pragma unroll
  for (int i = 0; i < kRateRows / 2 + 1; ++i) {
    const int64_t j = base + 2 * i + 1;
    nbs[i] = ev[i].yhat + ev[i + 1].yhat;
    od[i] = Out{0.f, 0.f, 0.f, 0.f};
    if (j >= 0 && j < P.N) od[i] = code_row(ys[2 * i + 1], us[2 * i + 1], fmaf(k.a, nbs[i], ms[2 * i + 1]), k, bad);
  }
#pragma unroll
  for (int i = 1; i <= kRateRows / 2; ++i) {
    const int64_t e = base + 2 * i, o = e + 1;
    const int le = 2 * i - 2;
    float be = 0.f, bo = 0.f;
    if (e < P.N) {
      const int64_t eo = e * kC + c;
      P.yhat[eo] = ev[i].yhat;
      // the even row's reconstruction feeds the means of rows e - 1 and e + 1
      P.gy[eo] = fmaf(k.a, -(od[i - 1].beta + od[i].beta) * inv_d, ev[i].beta * inv_d);
      P.gm[eo] = -ev[i].beta * inv_d;
      gb += (double)ev[i].gamma * (double)inv_d;
      be = ev[i].bits;
    }
    if (o < P.N) {
      const int64_t oo = o * kC + c;
      const float gmo = -od[i].beta * inv_d;
      P.yhat[oo] = od[i].yhat;
      P.gy[oo] = od[i].beta * inv_d;
      P.gm[oo] = gmo;
      ga += (double)gmo * (double)nbs[i];
      gb += (double)od[i].gamma * (double)inv_d;
      bo = od[i].bits;
    }
    lb[le * kRateCols + lt] = be;
    lb[(le + 1) * kRateCols + lt] = bo;
  }
  __syncthreads();
  // per-token bits of this block's columns: 16 lanes per row, 16 columns each
  {
    const int row = lt >> 4, part = lt & 15;
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < kRateCols / 16; ++q) sum += lb[row * kRateCols + q * 16 + part];
    sum = wave_sum16(sum);
    if (part == 0 && j0 + row < P.N) P.bits_part[cb * P.N + j0 + row] = sum;
  }
  P.ga_part[(int64_t)chunk * kC + c] = (float)ga;
  P.gb_part[(int64_t)chunk * kC + c] = (float)gb;
  const int any = __syncthreads_or(bad ? 1 : 0);
  if (lt == 0) P.flags[t] = any;
}

constexpr int kParCols = 64;              // components per reduction workgroup (one wave's row)
constexpr int kParGroups = 256 / kParCols;  // partial rows summed side by side
constexpr int kParSeg = 64;               // partial rows per first-stage workgroup

// The reductions after k_rate, by workgroup:
//   [0, nb)            per-token bits of 256 rows: the column-block partials in
//                      a fixed order; and the OR of the bad-input flags of the
//                      chunks those rows fall in
//   [nb, nb + C/64 S)  first stage of dR/da and dR/db: 64 components x one
//                      segment of kParSeg partial rows, summed by 4 groups
//                      (row i in group i % 4) in fp64, then the groups in order
struct FinishP {
  const float *bits_part;
  const float *ga_part, *gb_part;
  double *ga_seg, *gb_seg;  // [S][C]
  const int32_t *flags;
  int32_t *flags2;          // [nb]
  float *bits, *ga, *gb;
  int32_t *status;
  int64_t N, parts, n_flags;
  int nb, n_seg;
};

__global__ __launch_bounds__(256) void k_rate_finish(FinishP P) {
  __shared__ double sa[kParGroups][kParCols], sb[kParGroups][kParCols];
  const int b = blockIdx.x;
  if (b < P.nb) {
    const int64_t j = (int64_t)b * 256 + threadIdx.x;
    if (j < P.N) {
      float s = 0.f;
      for (int w = 0; w < kRateParts; ++w) s += P.bits_part[w * P.N + j];
      P.bits[j] = s;
    }
    // flags of chunks [16 b, 16 b + 16): (chunk, column block) pairs at t = 8 chunk + cb
    const int64_t f = (int64_t)b * (256 / kRateRows) * kRateParts + threadIdx.x;
    const int any = __syncthreads_or(threadIdx.x < (256 / kRateRows) * kRateParts && f < P.n_flags ? P.flags[f] : 0);
    if (threadIdx.x == 0) P.flags2[b] = any;
    return;
  }
  const int bb = b - P.nb;
  const int cg = bb % (kC / kParCols), seg = bb / (kC / kParCols);
  const int col = threadIdx.x % kParCols, grp = threadIdx.x / kParCols;
  const int c = cg * kParCols + col;
  const int64_t lo = (int64_t)seg * kParSeg, hi = min(lo + kParSeg, P.parts);
  double a = 0.0, g = 0.0;
  for (int64_t i = lo + grp; i < hi; i += kParGroups) {
    a += P.ga_part[i * kC + c];
    g += P.gb_part[i * kC + c];
  }
  sa[grp][col] = a;
  sb[grp][col] = g;
  __syncthreads();
  if (threadIdx.x < kParCols) {
    double ta = 0.0, tb = 0.0;
    for (int k = 0; k < kParGroups; ++k) {
      ta += sa[k][threadIdx.x];
      tb += sb[k][threadIdx.x];
    }
    P.ga_seg[(int64_t)seg * kC + c] = ta;
    P.gb_seg[(int64_t)seg * kC + c] = tb;
  }
}

// Second stage: workgroups [0, C / 64) add the segments of 64 components (4
// groups, segment i in group i % 4, then the groups in order); workgroup C / 64
// sets the status: EINVAL if any k_rate workgroup saw a bad input.
__global__ __launch_bounds__(256) void k_rate_finish2(FinishP P) {
  __shared__ double sa[kParGroups][kParCols], sb[kParGroups][kParCols];
  if (blockIdx.x < kC / kParCols) {
    const int col = threadIdx.x % kParCols, grp = threadIdx.x / kParCols;
    const int c = blockIdx.x * kParCols + col;
    double a = 0.0, g = 0.0;
    for (int i = grp; i < P.n_seg; i += kParGroups) {
      a += P.ga_seg[(int64_t)i * kC + c];
      g += P.gb_seg[(int64_t)i * kC + c];
    }
    sa[grp][col] = a;
    sb[grp][col] = g;
    __syncthreads();
    if (threadIdx.x < kParCols) {
      double ta = 0.0, tb = 0.0;
      for (int k = 0; k < kParGroups; ++k) {
        ta += sa[k][threadIdx.x];
        tb += sb[k][threadIdx.x];
      }
      P.ga[c] = (float)ta;
      P.gb[c] = (float)tb;
    }
    return;
  }
  int any = 0;
  for (int i = threadIdx.x; i < P.nb; i += 256) any |= P.flags2[i];
  any = __syncthreads_or(any);
  if (threadIdx.x == 0) *P.status = any ? DCKV_EINVAL : 0;
}

// k-slices of the transform: two when its tiles fill at most half of the 256
// compute units (k_rate adds at most two partial sets)
int rate_ksplit(int64_t N) {
  const int64_t tiles = ((N + kBM - 1) / kBM) * (kC / kBN);
  return tiles * 2 <= 256 ? 2 : 1;
}

// Xt[d][j] = rows[keep_head + j][d] for j < N, 0 for N <= j < n_pad (bf16,
// transposed through a 64 x 64 LDS tile with 8-byte accesses: 16 threads per
// 64-element row, 16 rows per pass)
__global__ __launch_bounds__(256) void k_rate_rows_t(const uint16_t *X, int64_t N, int64_t n_pad, uint16_t *Xt) {
  __shared__ uint16_t t[64][72];
  const int64_t j0 = (int64_t)blockIdx.x * 64;
  const int d0 = blockIdx.y * 64;
  const int q = threadIdx.x & 15, r = threadIdx.x >> 4;
  for (int p = 0; p < 4; ++p) {
    const int jr = r + 16 * p;
    const int64_t j = j0 + jr;
    uint2 v = make_uint2(0u, 0u);
    if (j < N) v = *reinterpret_cast<const uint2 *>(X + j * kD + d0 + 4 * q);
    *reinterpret_cast<uint2 *>(&t[jr][4 * q]) = v;
  }
  __syncthreads();
  for (int p = 0; p < 4; ++p) {
    const int dr = r + 16 * p;
    const uint32_t a = (uint32_t)t[4 * q][dr] | ((uint32_t)t[4 * q + 1][dr] << 16);
    const uint32_t b = (uint32_t)t[4 * q + 2][dr] | ((uint32_t)t[4 * q + 3][dr] << 16);
    *reinterpret_cast<uint2 *>(Xt + (int64_t)(d0 + dr) * n_pad + j0 + 4 * q) = make_uint2(a, b);
  }
}

__global__ __launch_bounds__(256) void k_rate_zero(float *p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

}  // namespace

RateBwdLayout rate_bwd_layout(int64_t N) {
  RateBwdLayout l;
  l.n_pad = (N + 63) / 64 * 64;
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t o = off;
    off = (off + bytes + 255) & ~(uint64_t)255;
    return o;
  };
  const uint64_t np = (uint64_t)l.n_pad;
  l.gy_hi = take(np * kC * 2);
  l.gy_lo = take(np * kC * 2);
  l.gm_hi = take(np * kC * 2);
  l.gm_lo = take(np * kC * 2);
  l.Xt = take(np * kD * 2);
  l.Et = take(np * kEmb * 2);
  l.tokc = take(np * 4);
  l.total = std::max<uint64_t>(off, 256);
  return l;
}

// dR/dA[c][d] = sum_j G_y[j][c] x_j[d] and dR/dH[c][e] = sum_j G_m[j][c] E[tok_j][e]
// on the fp32-output MFMA GEMM: the gradients enter as transposed bf16 high and
// low halves (16 mantissa bits) over two k ranges against the same transposed
// bf16 rows / gathered embeddings, so the products of the halves add up.
void rate_bwd_sequence(const RateBwdArgs &a) {
  const dckv_plan_t *p = a.p;
  const hipStream_t s = a.s;
  const RateBwdLayout &l = a.l;
  launch_clear_status(a.status, s);
  if (a.N == 0) {  // (a fill kernel, not a memset: the sequence may be captured in a graph)
    hipLaunchKernelGGL(k_rate_zero, dim3(1024), dim3(256), 0, s, a.grad_A, (int64_t)kC * kD);
    hipLaunchKernelGGL(k_rate_zero, dim3(256), dim3(256), 0, s, a.grad_H, (int64_t)kC * kEmb);
    return;
  }
  const int64_t np = l.n_pad;
  uint16_t *gy_hi = reinterpret_cast<uint16_t *>(a.ws + l.gy_hi), *gy_lo = reinterpret_cast<uint16_t *>(a.ws + l.gy_lo);
  uint16_t *gm_hi = reinterpret_cast<uint16_t *>(a.ws + l.gm_hi), *gm_lo = reinterpret_cast<uint16_t *>(a.ws + l.gm_lo);
  uint16_t *Xt = reinterpret_cast<uint16_t *>(a.ws + l.Xt), *Et = reinterpret_cast<uint16_t *>(a.ws + l.Et);
  int32_t *tokc = reinterpret_cast<int32_t *>(a.ws + l.tokc);
  launch_split_t(a.grad_y, a.N, np, gy_hi, gy_lo, s);
  launch_split_t(a.grad_mean, a.N, np, gm_hi, gm_lo, s);
  hipLaunchKernelGGL(k_rate_rows_t, dim3((unsigned)(np / 64), kD / 64), dim3(256), 0, s,
                     a.rows + (size_t)p->keep_head * kD, a.N, np, Xt);
  launch_gather_t(p->E, a.tok + p->keep_head, a.N, np, p->vocab, Et, tokc, a.status, s);
  GemmF32Args g{};
  g.a0 = gy_hi;
  g.a1 = gy_lo;
  g.lda0 = g.lda1 = (uint32_t)(np * 2);
  g.b0 = g.b1 = Xt;
  g.ldb0 = g.ldb1 = (uint32_t)(np * 2);
  g.split = (int)(np / kBK);
  g.KT = 2 * g.split;
  g.arow = nullptr;
  g.M = kC;
  g.N = kD;
  g.c = a.grad_A;
  g.ldc = kD;
  GemmF32Args h = g;
  h.a0 = gm_hi;
  h.a1 = gm_lo;
  h.b0 = h.b1 = Et;
  h.N = kEmb;
  h.c = a.grad_H;
  h.ldc = kEmb;
  // 192 + 64 tiles of the same depth: one launch fills the 256 compute units
  launch_gemm_f32_pair(g, h, s);
}

RateLayout rate_layout(int64_t N) {
  RateLayout l;
  l.chunks = (N + kRateRows - 1) / kRateRows;
  l.parts = l.chunks;
  l.ksplit = rate_ksplit(N);
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t o = off;
    off = (off + bytes + 255) & ~(uint64_t)255;
    return o;
  };
  l.Y = take((uint64_t)l.ksplit * N * kC * 4);
  l.bits_part = take((uint64_t)kRateParts * N * 4);
  l.ga_part = take((uint64_t)l.parts * kC * 4);
  l.gb_part = take((uint64_t)l.parts * kC * 4);
  l.flags = take((uint64_t)l.parts * (kC / kRateCols) * 4);
  l.n_seg = (l.parts + kParSeg - 1) / kParSeg;
  l.ga_seg = take((uint64_t)l.n_seg * kC * 8);
  l.gb_seg = take((uint64_t)l.n_seg * kC * 8);
  l.flags2 = take((uint64_t)(N + 255) / 256 * 4);
  l.total = std::max<uint64_t>(off, 256);
  return l;
}

void rate_sequence(const RateArgs &a) {
  const dckv_plan_t *p = a.p;
  const hipStream_t s = a.s;
  const RateLayout &l = a.l;
  float *ga_part = reinterpret_cast<float *>(a.ws + l.ga_part);
  float *gb_part = reinterpret_cast<float *>(a.ws + l.gb_part);
  if (a.N > 0) {
    float *Y = reinterpret_cast<float *>(a.ws + l.Y);
    GemmF32Args g{};
    g.a0 = g.a1 = a.rows + (size_t)p->keep_head * kD;
    g.lda0 = g.lda1 = kD * 2;
    g.b0 = g.b1 = p->A;
    g.ldb0 = g.ldb1 = kD * 2;
    g.KT = g.split = kD / kBK;
    g.arow = nullptr;
    g.M = (int)a.N;
    g.N = kC;
    g.c = Y;
    g.ldc = kC;
    g.ksplit = l.ksplit;
    launch_gemm_f32(g, s);
    RateP P;
    P.Y = Y;
    P.mtab = p->mtab;
    P.tok = a.tok;
    P.noise = a.noise;
    P.step = p->dev.step;
    P.nbr = p->dev.nbr;
    P.scale = p->dev.scale;
    P.rank = p->dev.rank;
    P.colpos = p->dev.colpos;
    P.yhat = a.yhat;
    P.gy = a.grad_y;
    P.gm = a.grad_mean;
    P.bits_part = reinterpret_cast<float *>(a.ws + l.bits_part);
    P.ga_part = ga_part;
    P.gb_part = gb_part;
    P.flags = reinterpret_cast<int32_t *>(a.ws + l.flags);
    P.N = a.N;
    P.keep_head = p->keep_head;
    P.vocab = p->vocab;
    P.ksplit = l.ksplit;
    P.chunks = l.chunks;
    {
      KernelTimer tm("rate", s);
      hipLaunchKernelGGL(k_rate, dim3((unsigned)(l.chunks * kRateParts)), dim3(kRateCols), 0, s, P);
    }
  }
  FinishP F;
  F.bits_part = reinterpret_cast<const float *>(a.ws + l.bits_part);
  F.ga_part = ga_part;
  F.gb_part = gb_part;
  F.flags = reinterpret_cast<const int32_t *>(a.ws + l.flags);
  F.bits = a.bits;
  F.ga = a.grad_nbr;
  F.gb = a.grad_scale;
  F.status = a.status;
  F.N = a.N;
  F.parts = l.parts;
  F.n_flags = l.parts * (kC / kRateCols);
  F.nb = (int)((a.N + 255) / 256);
  F.n_seg = (int)l.n_seg;
  F.ga_seg = reinterpret_cast<double *>(a.ws + l.ga_seg);
  F.gb_seg = reinterpret_cast<double *>(a.ws + l.gb_seg);
  F.flags2 = reinterpret_cast<int32_t *>(a.ws + l.flags2);
  const unsigned g1 = (unsigned)(F.nb + (kC / kParCols) * l.n_seg);
  if (g1 > 0) hipLaunchKernelGGL(k_rate_finish, dim3(g1), dim3(256), 0, s, F);
  hipLaunchKernelGGL(k_rate_finish2, dim3(kC / kParCols + 1), dim3(256), 0, s, F);
}

}  // namespace dckv
