// The first kernel of an encode: per-call initialisation and the kept-row
// copy (DCKV digest page, "How it works", first paragraph: the first 4 and
// last 128 positions stay in bf16).
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

}  // namespace

void launch_start_encode(const EncodeArgs &a) {
  const int64_t head_n = std::min<int64_t>(a.p->keep_head, a.g.T);
  hipLaunchKernelGGL(k_start_encode, dim3((unsigned)std::max<int64_t>(a.g.n_kept, 1)), dim3(256), 0, a.s, a.ws,
                     a.status, a.stream_bytes, a.rows, a.stream + kHeaderBytes, (int64_t)a.p->D, head_n,
                     (int64_t)a.p->keep_head + a.g.N, a.g.n_kept);
}

}  // namespace dckv
