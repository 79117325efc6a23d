// The first kernel of an encode: per-call initialisation and the kept-row
// copy (DCKV digest page, "How it works", first paragraph: the first 4 and
// last 128 positions stay in bf16).  Also the inverse RoPE that takes a
// post-RoPE cache back to the pre-RoPE rows the codec codes (same paragraph:
// keys are taken before RoPE).
#include "dckv_internal.h"

namespace dckv {
namespace {

// The start of an encode: workgroup 0 clears the control words, the status
// and the stream size; workgroup k (< n_kept) copies kept row k (first
// keep_head and last keep_tail positions) into the stream, verbatim and in
// position order, as 16-byte vectors (rows and stream are 16-byte aligned,
// rows are D * 2 bytes).
__global__ __launch_bounds__(256) void k_start_encode(uint8_t *ws, int32_t *status, uint64_t *stream_bytes,
                                                      const uint16_t *rows, uint8_t *dst, int64_t D, int64_t head_n,
                                                      int64_t tail_row0, int64_t n_kept) {
  const int64_t k = blockIdx.x;
  if (k == 0 && threadIdx.x == 0) {
    Ctrl *ct = reinterpret_cast<Ctrl *>(ws);
    ct->n_esc = 0;
    ct->status = 0;
    ct->total_bytes = 0;
    ct->rans_bytes = 0;
    ct->esc_off = ct->rans_off = ct->offs_off = 0;
    *status = 0;
    *stream_bytes = 0;
  }
  if (k >= n_kept) return;
  const int64_t src_row = k < head_n ? k : tail_row0 + (k - head_n);
  const uint4 *src = reinterpret_cast<const uint4 *>(rows + src_row * D);
  uint4 *out = reinterpret_cast<uint4 *>(dst + k * D * 2);
  for (int64_t i = threadIdx.x; i < D / 8; i += blockDim.x) out[i] = src[i];
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
}  // namespace

void launch_start_encode(const EncodeArgs &a) {
  const int64_t head_n = std::min<int64_t>(a.p->keep_head, a.g.T);
  hipLaunchKernelGGL(k_start_encode, dim3((unsigned)std::max<int64_t>(a.g.n_kept, 1)), dim3(256), 0, a.s, a.ws,
                     a.status, a.stream_bytes, a.rows, a.stream + kHeaderBytes, (int64_t)a.p->D, head_n,
                     (int64_t)a.p->keep_head + a.g.N, a.g.n_kept);
}

}  // namespace dckv

namespace dckv {
void launch_unrope(const dckv_plan_t *p, const uint16_t *in, uint16_t *out, int64_t T, hipStream_t s) {
  if (T == 0) return;
  hipLaunchKernelGGL(k_unrope, dim3((unsigned)((T + 1) / 2)), dim3(256), 0, s, in, out, T, p->dev.omega);
}
}  // namespace dckv
