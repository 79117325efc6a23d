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
  const int32_t *pre;  // set: the status starts as *pre
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
    *P.status = P.pre ? *P.pre : 0;
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
// caller's rows where they are.  Thread (row t, group g) takes frequencies
// 8 g .. 8 g + 7 of every key head: one angle computation per frequency for
// all 12 heads, and 16-byte loads and stores.  Same fp64 arithmetic as
// k_unrope, so the copy's keys equal its output bit for bit.
__global__ __launch_bounds__(256) void k_unrope_keys(const uint16_t *in, uint16_t *kc, int64_t T,
                                                     const double *omega) {
  const int64_t t = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int g = threadIdx.x & 15;
  if (t >= T) return;
  double cs[8], sn[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sincos((double)t * omega[8 * g + e], &sn[e], &cs[e]);
  const uint16_t *src = in + (size_t)t * kD;
  uint16_t *dst = kc + (size_t)t * kKeyCols;
  auto lanes = [](const uint4 &v, int e) -> uint32_t {
    const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return (e & 1) ? w >> 16 : w & 0xFFFFu;
  };
#pragma unroll
  for (int l = 0; l < 6; ++l)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kb = (l * 4 + h) * kHeadDim + 8 * g, ob = (l * 2 + h) * kHeadDim + 8 * g;
      const uint4 a = *reinterpret_cast<const uint4 *>(src + kb);
      const uint4 b = *reinterpret_cast<const uint4 *>(src + kb + kHalf);
      uint32_t o0[4], o1[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        uint32_t r0[2], r1[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const double p0 = (double)__uint_as_float(lanes(a, e + u) << 16);
          const double p1 = (double)__uint_as_float(lanes(b, e + u) << 16);
          r0[u] = bf16_of_f64(__dadd_rn(__dmul_rn(p0, cs[e + u]), __dmul_rn(p1, sn[e + u])));
          r1[u] = bf16_of_f64(__dsub_rn(__dmul_rn(p1, cs[e + u]), __dmul_rn(p0, sn[e + u])));
        }
        o0[e / 2] = r0[0] | (r0[1] << 16);
        o1[e / 2] = r1[0] | (r1[1] << 16);
      }
      *reinterpret_cast<uint4 *>(dst + ob) = uint4{o0[0], o0[1], o0[2], o0[3]};
      *reinterpret_cast<uint4 *>(dst + ob + kHalf) = uint4{o1[0], o1[1], o1[2], o1[3]};
    }
}
// ---------------------------------------------------------------------------
// Paged attention cache (the layout serving engines keep the cache in): per
// layer a key and a value pool of [n_blocks][block_size][n_kv_heads][head_dim]
// bf16 and one block table for the request.  Position t is row
// table[t / bs] * bs + t % bs of every pool; its 6,144-dim codec row is, per
// layer l, the key heads then the value heads.
// ---------------------------------------------------------------------------

// Every entry of the request's block table in [0, n_blocks), else EINVAL.
// One workgroup: thread 0 clears the word first when asked, the others wait.
__global__ __launch_bounds__(256) void k_paged_check(const int32_t *table, int64_t n_logical, int64_t n_blocks,
                                                     int32_t *status, int clear_first) {
  if (clear_first) {
    if (threadIdx.x == 0) *status = 0;
    __syncthreads();
  }
  for (int64_t i = threadIdx.x; i < n_logical; i += blockDim.x) {
    const int64_t b = table[i];
    if (b < 0 || b >= n_blocks) atomicCAS(status, 0, DCKV_EINVAL);
  }
}

// row t (thread group of 16 per row) from the pools; thread g takes the
// 16-byte pieces 8 g .. 8 g + 7 of each half of every head, so a key pair
// (d, d + 128) is one thread's (the inverse rotation as k_unrope_keys)
__global__ __launch_bounds__(256) void k_paged_gather(PagedKV kv, int post_rope, int64_t T, const double *omega,
                                                      uint16_t *rows, const int32_t *pre) {
  const int64_t t = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int g = threadIdx.x & 15;
  if (t >= T || *pre != 0) return;
  const int64_t prow = (int64_t)kv.table[t / kv.bs] * kv.bs + t % kv.bs;
  double cs[8], sn[8];
  if (post_rope) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sincos((double)t * omega[8 * g + e], &sn[e], &cs[e]);
  }
  uint16_t *dst = rows + (size_t)t * kD;
  auto half = [](const uint4 &v, int e) -> uint32_t {
    const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return (e & 1) ? w >> 16 : w & 0xFFFFu;
  };
#pragma unroll
  for (int l = 0; l < 6; ++l)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const size_t so = ((size_t)prow * 2 + h) * kHeadDim + 8 * g;
      const uint16_t *ks = kv.p[2 * l] + so, *vs = kv.p[2 * l + 1] + so;
      const int kb = (l * 4 + h) * kHeadDim + 8 * g, vb = (l * 4 + 2 + h) * kHeadDim + 8 * g;
      const uint4 a = *reinterpret_cast<const uint4 *>(ks), b = *reinterpret_cast<const uint4 *>(ks + kHalf);
      *reinterpret_cast<uint4 *>(dst + vb) = *reinterpret_cast<const uint4 *>(vs);
      *reinterpret_cast<uint4 *>(dst + vb + kHalf) = *reinterpret_cast<const uint4 *>(vs + kHalf);
      if (!post_rope) {
        *reinterpret_cast<uint4 *>(dst + kb) = a;
        *reinterpret_cast<uint4 *>(dst + kb + kHalf) = b;
        continue;
      }
      uint32_t o0[4], o1[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        uint32_t r0[2], r1[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const double p0 = (double)__uint_as_float(half(a, e + u) << 16);
          const double p1 = (double)__uint_as_float(half(b, e + u) << 16);
          r0[u] = bf16_of_f64(__dadd_rn(__dmul_rn(p0, cs[e + u]), __dmul_rn(p1, sn[e + u])));
          r1[u] = bf16_of_f64(__dsub_rn(__dmul_rn(p1, cs[e + u]), __dmul_rn(p0, sn[e + u])));
        }
        o0[e / 2] = r0[0] | (r0[1] << 16);
        o1[e / 2] = r1[0] | (r1[1] << 16);
      }
      *reinterpret_cast<uint4 *>(dst + kb) = uint4{o0[0], o0[1], o0[2], o0[3]};
      *reinterpret_cast<uint4 *>(dst + kb + kHalf) = uint4{o1[0], o1[1], o1[2], o1[3]};
    }
}

// the pools from rows: thread (t, 16-byte piece i) of a row's 768 pieces
__global__ __launch_bounds__(256) void k_paged_scatter(PagedKV kv, int64_t T, const uint16_t *rows,
                                                       const int32_t *status) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * (kD / 8) || *status != 0) return;
  const int64_t t = i / (kD / 8);
  const int c = (int)(i - t * (kD / 8)) * 8;  // column of the piece
  const int l = c / 1024, w = c % 1024, kvi = w / 512, h = (w % 512) / kHeadDim, d = w % kHeadDim;
  const int64_t prow = (int64_t)kv.table[t / kv.bs] * kv.bs + t % kv.bs;
  *reinterpret_cast<uint4 *>(kv.p[2 * l + kvi] + ((size_t)prow * 2 + h) * kHeadDim + d) =
      *reinterpret_cast<const uint4 *>(rows + (size_t)t * kD + c);
}
}  // namespace

void launch_start_encode(const EncodeArgs *args, int n) {
  auto fill = [&](int i) {
    const EncodeArgs &a = args[i];
    StartP P;
    P.ws = a.ws;
    P.status = a.status;
    P.pre = a.pre;
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
  hipLaunchKernelGGL(k_unrope_keys, dim3((unsigned)((T + 15) / 16)), dim3(256), 0, s, in, kc, T, p->dev.omega);
}

void launch_unrope(const dckv_plan_t *p, const uint16_t *in, uint16_t *out, int64_t T, hipStream_t s) {
  if (T == 0) return;
  hipLaunchKernelGGL(k_unrope, dim3((unsigned)((T + 1) / 2)), dim3(256), 0, s, in, out, T, p->dev.omega);
}
void launch_paged_check(const PagedKV &kv, int64_t T, int32_t *status, bool clear_first, hipStream_t s) {
  const int64_t n_logical = T > 0 ? (T + kv.bs - 1) / kv.bs : 0;
  hipLaunchKernelGGL(k_paged_check, dim3(1), dim3(256), 0, s, kv.table, n_logical, kv.n_blocks, status,
                     clear_first ? 1 : 0);
}

void launch_paged_gather(const dckv_plan_t *p, const PagedKV &kv, bool post_rope, int64_t T, uint16_t *rows,
                         const int32_t *pre, hipStream_t s) {
  if (T <= 0) return;
  KernelTimer tm("paged_gather", s);
  hipLaunchKernelGGL(k_paged_gather, dim3((unsigned)((T + 15) / 16)), dim3(256), 0, s, kv, post_rope ? 1 : 0, T,
                     p->dev.omega, rows, pre);
}

void launch_paged_scatter(const PagedKV &kv, int64_t T, const uint16_t *rows, const int32_t *status, hipStream_t s) {
  if (T <= 0) return;
  KernelTimer tm("paged_scatter", s);
  const int64_t n = T * (kD / 8);
  hipLaunchKernelGGL(k_paged_scatter, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, kv, T, rows, status);
}
}  // namespace dckv
