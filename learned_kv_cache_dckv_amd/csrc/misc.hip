// The first kernel of an encode: per-call initialisation and the kept-row
// copy (DCKV digest page, "How it works", first paragraph: the first 4 and
// last 128 positions stay in bf16).  Also the inverse RoPE that takes a
// post-RoPE cache back to the pre-RoPE rows the codec codes (same paragraph:
// the codec sees the keys without their rotary embedding).
#include "dckv_internal.h"

namespace dckv {
namespace {

// The start of an encode: workgroup 0 clears the control words, the status
// and the stream size; workgroup k (< n_kept) copies kept row k (first
// keep_head and last keep_tail positions) into the stream, verbatim and in
// position order, as 16-byte vectors (rows and stream are 16-byte aligned,
// rows are D * 2 bytes).
struct StartP {
  uint8_t *ws;
  int32_t *status;
  uint64_t *stream_bytes;
  const uint16_t *rows;
  const uint16_t *keys;  // set: the key heads of every row come from this key copy [T][kKeyCols]
  uint8_t *dst;
  int64_t D, head_n, tail_row0, n_kept;
};

__global__ __launch_bounds__(256) void k_start_encode(const Batch<StartP> B) {
  const int ri = batch_req(B, blockIdx.x);
  const StartP &P = B.r[ri];
  const int64_t k = blockIdx.x - B.start[ri];
  if (k == 0 && threadIdx.x == 0) {
    Ctrl *ct = reinterpret_cast<Ctrl *>(P.ws);
    ct->n_esc = 0;
    ct->status = 0;
    ct->total_bytes = 0;
    ct->rans_bytes = 0;
    ct->esc_off = ct->rans_off = ct->offs_off = 0;
    *P.status = 0;
    *P.stream_bytes = 0;
  }
  if (k >= P.n_kept) return;
  const int64_t src_row = k < P.head_n ? k : P.tail_row0 + (k - P.head_n);
  const uint4 *src = reinterpret_cast<const uint4 *>(P.rows + src_row * P.D);
  uint4 *out = reinterpret_cast<uint4 *>(P.dst + k * P.D * 2);
  if (!P.keys) {
    for (int64_t i = threadIdx.x; i < P.D / 8; i += blockDim.x) out[i] = src[i];
    return;
  }
  // 16-byte piece i of the row is in head block i / 32 (4 per layer: key
  // heads 0, 1, value heads 0, 1); key pieces come from the key copy
  const uint4 *ksrc = reinterpret_cast<const uint4 *>(P.keys + src_row * kKeyCols);
  for (int64_t i = threadIdx.x; i < P.D / 8; i += blockDim.x) {
    const int64_t blk = i >> 5;
    out[i] = (blk & 2) ? src[i] : ksrc[((blk >> 2) * 2 + (blk & 1)) * 32 + (i & 31)];
  }
}

// bf16 of a double, one correct rounding to nearest even: truncate to fp32,
// mark an inexact truncation in the lowest bit (round to odd), then round
// the 32-bit pattern to 16 bits
__device__ __forceinline__ uint16_t bf16_of_f64(double x) {
  const float f = __double2float_rz(x);
  uint32_t u = __float_as_uint(f);
  if ((double)f != x) u |= 1u;
  if (isnan(x)) return 0x7FC0;
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Inverse RoPE of row t (blockIdx.x * 2 + thread / 128) on the key heads,
// frequency d = thread % 128: (x0, x1) = (p0 c + p1 s, p1 c - p0 s) in fp64
// (no fused products) at angle t w_d; value heads are copied.
__global__ __launch_bounds__(256) void k_unrope(const uint16_t *in, uint16_t *out, int64_t T, const double *omega) {
  const int64_t t = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 7);
  const int d = threadIdx.x & 127;
  if (t >= T) return;
  double sn, cs;
  sincos((double)t * omega[d], &sn, &cs);
  const uint16_t *src = in + (size_t)t * kD;
  uint16_t *dst = out + (size_t)t * kD;
#pragma unroll
  for (int l = 0; l < 6; ++l)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kb = (l * 4 + h) * kHeadDim, vb = (l * 4 + 2 + h) * kHeadDim;
      const double p0 = (double)__uint_as_float((uint32_t)src[kb + d] << 16);
      const double p1 = (double)__uint_as_float((uint32_t)src[kb + d + kHalf] << 16);
      const uint16_t v0 = src[vb + d], v1 = src[vb + d + kHalf];
      dst[kb + d] = bf16_of_f64(__dadd_rn(__dmul_rn(p0, cs), __dmul_rn(p1, sn)));
      dst[kb + d + kHalf] = bf16_of_f64(__dsub_rn(__dmul_rn(p1, cs), __dmul_rn(p0, sn)));
      dst[vb + d] = v0;
      dst[vb + d + kHalf] = v1;
    }
}

// The same inverse rotation of the key heads only, into the key copy
// kc [T][6 * 2 * head_dim] (layer l, head h at columns (l * 2 + h) * head_dim):
// half the traffic of a whole-row pass; the value heads are read from the
// caller's rows where they are.
__global__ __launch_bounds__(256) void k_unrope_keys(const uint16_t *in, uint16_t *kc, int64_t T,
                                                     const double *omega) {
  const int64_t t = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 7);
  const int d = threadIdx.x & 127;
  if (t >= T) return;
  double sn, cs;
  sincos((double)t * omega[d], &sn, &cs);
  const uint16_t *src = in + (size_t)t * kD;
  uint16_t *dst = kc + (size_t)t * kKeyCols;
#pragma unroll
  for (int l = 0; l < 6; ++l)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kb = (l * 4 + h) * kHeadDim, ob = (l * 2 + h) * kHeadDim;
      const double p0 = (double)__uint_as_float((uint32_t)src[kb + d] << 16);
      const double p1 = (double)__uint_as_float((uint32_t)src[kb + d + kHalf] << 16);
      dst[ob + d] = bf16_of_f64(__dadd_rn(__dmul_rn(p0, cs), __dmul_rn(p1, sn)));
      dst[ob + d + kHalf] = bf16_of_f64(__dsub_rn(__dmul_rn(p1, cs), __dmul_rn(p0, sn)));
    }
}
}  // namespace

void launch_start_encode(const EncodeArgs *args, int n) {
  auto fill = [&](int i) {
    const EncodeArgs &a = args[i];
    StartP P;
    P.ws = a.ws;
    P.status = a.status;
    P.stream_bytes = a.stream_bytes;
    P.rows = a.rows;
    P.keys = a.keys;
    P.dst = a.stream + kHeaderBytes;
    P.D = a.p->D;
    P.head_n = std::min<int64_t>(a.p->keep_head, a.g.T);
    P.tail_row0 = (int64_t)a.p->keep_head + a.g.N;
    P.n_kept = a.g.n_kept;
    return P;
  };
  auto count = [&](int i) { return (uint32_t)std::max<int64_t>(args[i].g.n_kept, 1); };
  launch_batched<StartP>(k_start_encode, "start", n, args[0].s, 256, fill, count);
}

void launch_unrope_keys(const dckv_plan_t *p, const uint16_t *in, uint16_t *kc, int64_t T, hipStream_t s) {
  if (T <= 0) return;
  KernelTimer tm("unrope_keys", s);
  hipLaunchKernelGGL(k_unrope_keys, dim3((unsigned)((T + 1) / 2)), dim3(256), 0, s, in, kc, T, p->dev.omega);
}

void launch_unrope(const dckv_plan_t *p, const uint16_t *in, uint16_t *out, int64_t T, hipStream_t s) {
  if (T == 0) return;
  hipLaunchKernelGGL(k_unrope, dim3((unsigned)((T + 1) / 2)), dim3(256), 0, s, in, out, T, p->dev.omega);
}
}  // namespace dckv
