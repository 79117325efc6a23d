// The rate term of codec training and its gradients (DCKV digest page, "How
// it works", Training bullet: code length computed with additive noise,
// reconstruction from rounded values with a straight-through gradient).
//
// For coded row j and active component c, with step D, Laplace scale b,
// s = b / D, neighbour weight a and embedding mean m:
//   even j: mu = m;  odd j: mu = m + a (yhat_{j-1} + yhat_{j+1}), yhat_N = 0
//   q = rint(fp32(y - mu) / D),  yhat = mu + q D     (the codec's two passes)
//   t = (y - mu) / D + u,        u the caller's noise in steps
//   bits = -log2(F_s(t + 1/2) - F_s(t - 1/2)),  F_s the zero-mean Laplace CDF
// and, with beta = d bits / dt and gamma = d bits / ds,
//   dR/dm_j = -beta_j / D
//   dR/dy_j = beta_j / D + [j even] a (dR/dm_{j-1} + dR/dm_{j+1})  (odd rows)
//   dR/da   = sum over odd j of dR/dm_j (yhat_{j-1} + yhat_{j+1})
//   dR/db   = sum over j of gamma_j / D.
// Dropped components: bits 0, yhat = mu, no gradient.
//
// Work split: the coefficients y = A x come from the fp32-output GEMM; one
// thread per component walks a chunk of rows in order, so the neighbour terms
// are register carries (two halo rows before the chunk and one after it are
// recomputed).  Per-token bits are wave sums written as partials and added in
// a fixed order; the per-component sums are per-chunk partials in fp64.
#include "dckv_internal.h"

namespace dckv {
namespace {

constexpr int kRateRows = 32;    // rows per chunk (even)
constexpr int kRateCols = 256;   // components per workgroup
constexpr int kRateWaves = kC / 64;  // wave partials per row

struct RateP {
  const float *Y;        // [N][C] coefficients
  const float *mtab;     // [vocab][C] embedding means, plan column order
  const int32_t *tok;    // [T]
  const float *noise;    // [N][C]
  const float *step, *nbr, *scale;
  const int32_t *rank, *colpos;
  float *yhat, *gy, *gm;  // [N][C]
  float *bits_part;       // [kRateWaves][N]
  double *ga_part, *gb_part;  // [chunks][C]
  int32_t *status;
  int64_t N;
  int keep_head, vocab;
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

struct Row {
  float y, m, u;
};

__device__ __forceinline__ Row load_row(const RateP &P, int64_t j, int c, const Col &k, bool &bad) {
  Row r;
  const int64_t o = j * kC + c;
  r.y = P.Y[o];
  r.u = P.noise[o];
  int v = P.tok[j + P.keep_head];
  if ((unsigned)v >= (unsigned)P.vocab) {
    bad = true;
    v = 0;
  }
  r.m = P.mtab[(int64_t)v * kC + k.col];
  return r;
}

// reconstruction and rate of one row given its conditional mean
__device__ __forceinline__ Out code_row(const Row &r, float mu, const Col &k, bool &bad) {
  Out o;
  if (!k.act) {
    o.yhat = mu;
    o.beta = o.gamma = o.bits = 0.f;
    return o;
  }
  const float d = r.y - mu;
  if (!isfinite(d)) bad = true;
  const float rr = __fdiv_rn(d, k.step);
  const float q = fminf(fmaxf(rintf(rr), -2147483520.0f), 2147483520.0f);
  o.yhat = fmaf(q, k.step, mu);
  rate_of(rr + r.u, k, o);
  return o;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__global__ __launch_bounds__(256) void k_rate(RateP P) {
  const int c = blockIdx.x * kRateCols + threadIdx.x;
  const int lane = threadIdx.x & 63;
  const int wv = c >> 6;
  const int64_t j0 = (int64_t)blockIdx.y * kRateRows;
  const int64_t j1 = min(j0 + kRateRows, P.N);
  Col k;
  k.step = P.step[c];
  k.a = P.nbr[c];
  k.act = P.rank[c] >= 0;
  k.col = P.colpos[c];
  k.s = P.scale[c] / k.step;
  k.inv_s_l2 = kLog2e / k.s;
  k.k0 = 1.f - log2f(-expm1f(-1.f / k.s));
  k.g0 = 1.f / expm1f(1.f / k.s);
  bool bad = false;
  double ga = 0.0, gb = 0.0;
  const float inv_d = 1.f / k.step;

  // the first even row, and the odd row before it (its dR/dm feeds the chain)
  const Row r0 = load_row(P, j0, c, k, bad);
  Out oe = code_row(r0, r0.m, k, bad);
  float gm_prev = 0.f;  // dR/dm of row j0 - 1
  if (j0 >= 2) {
    const Row rp = load_row(P, j0 - 2, c, k, bad);
    const Out op = code_row(rp, rp.m, k, bad);
    const Row ro = load_row(P, j0 - 1, c, k, bad);
    const Out oo = code_row(ro, fmaf(k.a, op.yhat + oe.yhat, ro.m), k, bad);
    gm_prev = -oo.beta * inv_d;
  }
  for (int64_t e = j0; e < j1; e += 2) {
    const int64_t o = e + 1;
    Out on = {0.f, 0.f, 0.f, 0.f};     // the odd row e + 1
    Out onext = {0.f, 0.f, 0.f, 0.f};  // the next even row e + 2
    bool have_next = false;
    if (o < P.N) {
      if (e + 2 < P.N) {
        const Row rn = load_row(P, e + 2, c, k, bad);
        onext = code_row(rn, rn.m, k, bad);
        have_next = true;
      }
      const Row ro = load_row(P, o, c, k, bad);
      const float nb = oe.yhat + (have_next ? onext.yhat : 0.f);
      const float mu = fmaf(k.a, nb, ro.m);
      on = code_row(ro, mu, k, bad);
      const float gmo = -on.beta * inv_d;
      ga += (double)gmo * (double)nb;
      gb += (double)on.gamma * (double)inv_d;
      const int64_t oo = o * kC + c;
      P.yhat[oo] = on.yhat;
      P.gy[oo] = on.beta * inv_d;
      P.gm[oo] = gmo;
    }
    // the even row: its reconstruction feeds the means of rows e - 1 and e + 1
    const float gme = -oe.beta * inv_d;
    const float gm_next = -on.beta * inv_d;
    const int64_t eo = e * kC + c;
    P.yhat[eo] = oe.yhat;
    P.gy[eo] = fmaf(k.a, gm_prev + gm_next, oe.beta * inv_d);
    P.gm[eo] = gme;
    gb += (double)oe.gamma * (double)inv_d;
    const float be = wave_sum(oe.bits);
    const float bo = wave_sum(on.bits);
    if (lane == 0) {
      P.bits_part[wv * P.N + e] = be;
      if (o < P.N) P.bits_part[wv * P.N + o] = bo;
    }
    gm_prev = gm_next;
    oe = onext;
  }
  P.ga_part[(int64_t)blockIdx.y * kC + c] = ga;
  P.gb_part[(int64_t)blockIdx.y * kC + c] = gb;
  if (bad) *P.status = DCKV_EINVAL;
}

// per-token bits: the wave partials in a fixed order
__global__ __launch_bounds__(256) void k_rate_bits(const float *part, int64_t N, float *bits) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= N) return;
  float s = 0.f;
  for (int w = 0; w < kRateWaves; ++w) s += part[w * N + j];
  bits[j] = s;
}

// per-component sums over the chunks
__global__ __launch_bounds__(256) void k_rate_params(const double *ga_part, const double *gb_part, int chunks,
                                                     float *ga, float *gb) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  double a = 0.0, b = 0.0;
  for (int i = 0; i < chunks; ++i) {
    a += ga_part[(int64_t)i * kC + c];
    b += gb_part[(int64_t)i * kC + c];
  }
  ga[c] = (float)a;
  gb[c] = (float)b;
}

__global__ void k_rate_clear_status(int32_t *status) { *status = 0; }

}  // namespace

RateLayout rate_layout(int64_t N) {
  RateLayout l;
  l.chunks = (N + kRateRows - 1) / kRateRows;
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t o = off;
    off = (off + bytes + 255) & ~(uint64_t)255;
    return o;
  };
  l.Y = take((uint64_t)N * kC * 4);
  l.bits_part = take((uint64_t)kRateWaves * N * 4);
  l.ga_part = take((uint64_t)l.chunks * kC * 8);
  l.gb_part = take((uint64_t)l.chunks * kC * 8);
  l.total = std::max<uint64_t>(off, 256);
  return l;
}

void rate_sequence(const RateArgs &a) {
  const dckv_plan_t *p = a.p;
  const hipStream_t s = a.s;
  hipLaunchKernelGGL(k_rate_clear_status, dim3(1), dim3(1), 0, s, a.status);
  const RateLayout &l = a.l;
  double *ga_part = reinterpret_cast<double *>(a.ws + l.ga_part);
  double *gb_part = reinterpret_cast<double *>(a.ws + l.gb_part);
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
    P.status = a.status;
    P.N = a.N;
    P.keep_head = p->keep_head;
    P.vocab = p->vocab;
    {
      KernelTimer tm("rate", s);
      hipLaunchKernelGGL(k_rate, dim3(kC / kRateCols, (unsigned)l.chunks), dim3(kRateCols), 0, s, P);
    }
    hipLaunchKernelGGL(k_rate_bits, dim3((unsigned)((a.N + 255) / 256)), dim3(256), 0, s, P.bits_part, a.N, a.bits);
  }
  hipLaunchKernelGGL(k_rate_params, dim3(kC / 256), dim3(256), 0, s, ga_part, gb_part, (int)l.chunks, a.grad_nbr,
                     a.grad_scale);
}

}  // namespace dckv
