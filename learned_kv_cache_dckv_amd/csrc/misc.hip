// Small kernels of the DCKV codec: per-call initialisation, the kept-row copy
// and the ordering of escape records.
//
// Escapes (DCKV digest page, "How it works", Coding bullet: codes beyond
// +-127 are escaped at 64 bits each) are found out of order by the quantiser
// tiles; the stream stores them by ascending flat index j * C_a + rank, so
// one workgroup sorts the (usually few) records with a bitonic network.
#include "dckv_internal.h"

namespace dckv {
namespace {

// The kept rows (first keep_head and last keep_tail positions) into the
// stream, verbatim and in position order: one workgroup per row, 16-byte
// vectors (rows and stream are 16-byte aligned, rows are D * 2 bytes).
__global__ __launch_bounds__(256) void k_kept_copy(const uint16_t *rows, uint8_t *dst, int64_t D, int64_t head_n,
                                                   int64_t tail_row0) {
  const int64_t k = blockIdx.x;
  const int64_t src_row = k < head_n ? k : tail_row0 + (k - head_n);
  const uint4 *src = reinterpret_cast<const uint4 *>(rows + src_row * D);
  uint4 *out = reinterpret_cast<uint4 *>(dst + k * D * 2);
  for (int64_t i = threadIdx.x; i < D / 8; i += blockDim.x) out[i] = src[i];
}

__global__ void k_init(uint8_t *ws, int32_t *status, uint64_t *stream_bytes) {
  if (threadIdx.x == 0) {
    Ctrl *ct = reinterpret_cast<Ctrl *>(ws);
    ct->n_esc = 0;
    ct->status = 0;
    ct->total_bytes = 0;
    ct->rans_bytes = 0;
    ct->esc_off = ct->rans_off = ct->offs_off = 0;
    *status = 0;
    if (stream_bytes) *stream_bytes = 0;
  }
}

constexpr int kSortLds = 4096;

__device__ __forceinline__ void bitonic(unsigned long long *a, uint32_t n_pow2) {
  for (uint32_t k = 2; k <= n_pow2; k <<= 1) {
    for (uint32_t j = k >> 1; j > 0; j >>= 1) {
      for (uint32_t i = threadIdx.x; i < n_pow2; i += blockDim.x) {
        const uint32_t l = i ^ j;
        if (l > i) {
          const unsigned long long x = a[i], y = a[l];
          const bool up = (i & k) == 0;
          if ((x > y) == up) {
            a[i] = y;
            a[l] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

// esc_raw holds {flat, q} pairs in arrival order; esc_sorted receives them by
// ascending flat.  esc_raw has room for the padded power-of-two count.
__global__ __launch_bounds__(1024) void k_esc_sort(uint8_t *ws, uint32_t *esc_raw, uint32_t *esc_sorted,
                                                   int64_t esc_cap, const int32_t *status) {
  __shared__ unsigned long long keys[kSortLds];
  if (*status != 0) return;
  const Ctrl *ct = reinterpret_cast<const Ctrl *>(ws);
  const uint32_t n = (uint32_t)min<int64_t>(ct->n_esc, esc_cap);
  if (n == 0) return;
  uint32_t p2 = 1;
  while (p2 < n) p2 <<= 1;
  unsigned long long *a;
  unsigned long long *g = reinterpret_cast<unsigned long long *>(esc_raw);
  if (p2 <= (uint32_t)kSortLds) {
    a = keys;
    for (uint32_t i = threadIdx.x; i < p2; i += blockDim.x)
      a[i] = i < n ? (((unsigned long long)esc_raw[2 * i]) << 32) | esc_raw[2 * i + 1] : ~0ull;
  } else {
    // in place in global memory: keys overwrite the pairs they were made from
    a = g;
    for (uint32_t i = threadIdx.x; i < p2; i += blockDim.x) {
      unsigned long long v = ~0ull;
      if (i < n) v = (((unsigned long long)esc_raw[2 * i]) << 32) | esc_raw[2 * i + 1];
      a[i] = v;  // element i occupies exactly the bytes of pair i
    }
  }
  __syncthreads();
  bitonic(a, p2);
  for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) {
    const unsigned long long v = a[i];
    esc_sorted[2 * i] = (uint32_t)(v >> 32);
    esc_sorted[2 * i + 1] = (uint32_t)v;
  }
}

}  // namespace

void launch_init(const EncodeArgs &a) {
  hipLaunchKernelGGL(k_init, dim3(1), dim3(64), 0, a.s, a.ws, a.status, a.stream_bytes);
}

void launch_init(const DecodeArgs &a) {
  hipLaunchKernelGGL(k_init, dim3(1), dim3(64), 0, a.s, a.ws, a.status, (uint64_t *)nullptr);
}

void launch_kept_copy(const EncodeArgs &a) {
  if (a.g.n_kept == 0) return;
  const int64_t head_n = std::min<int64_t>(a.p->keep_head, a.g.T);
  hipLaunchKernelGGL(k_kept_copy, dim3((unsigned)a.g.n_kept), dim3(256), 0, a.s, a.rows, a.stream + kHeaderBytes,
                     (int64_t)a.p->D, head_n, (int64_t)a.p->keep_head + a.g.N);
}

void launch_esc_sort(const EncodeArgs &a) {
  hipLaunchKernelGGL(k_esc_sort, dim3(1), dim3(1024), 0, a.s, a.ws,
                     reinterpret_cast<uint32_t *>(a.ws + a.l.esc_raw),
                     reinterpret_cast<uint32_t *>(a.ws + a.l.esc_sorted), a.g.esc_cap, a.status);
}

}  // namespace dckv
