// C ABI entry points of the DCKV codec: argument checks and the launch
// sequence of each call.  Every call only enqueues work on the caller's HIP
// stream; nothing here allocates device memory.
//
// Encode (DCKV digest page, "How it works"): control words and kept rows ->
// analysis GEMM with the quantiser (means from the plan's embedding-mean
// table; even rows, then odd rows with both reconstructed neighbours;
// escape records) -> fix-up of the odd row at each tile edge -> rANS per
// group -> escape sort, group offsets and header -> packing.
// Decode: parse and validate (and the RoPE tables) -> rANS per group -> the
// two dequantisation passes -> correction hidden layer (and RoPE of the kept
// rows) -> synthesis with RoPE.
// Fit (DCKV digest page, Evidence): the closed-form fit of the conditional
// models from calibration rows.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "dckv_internal.h"

using namespace dckv;

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_device(const dckv_plan_t *p) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return set_error(DCKV_EHIP, "no HIP device");
  if (cur != p->device) return set_error(DCKV_EINVAL, "the current HIP device is not the plan's device");
  return DCKV_OK;
}

// encode_only: the workspace need only hold what the encode kernels touch
int common_checks(const dckv_plan_t *p, int64_t T, void *ws, uint64_t ws_bytes, int32_t *status, Geometry &g,
                  Layout &l, bool encode_only = false) {
  if (!p) return set_error(DCKV_EINVAL, "null plan");
  if (T < 0 || T > 0x7FFFFFFF) return set_error(DCKV_EINVAL, "T out of range");
  if (T > kMaxRows) return set_error(DCKV_EUNSUPPORTED, "T above 2^18 positions (32-bit operand offsets)");
  if (!status || !aligned(status, 4)) return set_error(DCKV_EINVAL, "status must be a 4-byte aligned device word");
  if (!ws || !aligned(ws, 256)) return set_error(DCKV_EINVAL, "workspace must be 256-byte aligned");
  g = geometry(p, T);
  l = layout(p, g);
  if ((uint64_t)g.N * (uint64_t)std::max(p->C_a, 1) >= 0xFFFFFFFFull)
    return set_error(DCKV_EUNSUPPORTED, "request too long for 32-bit escape indices");
  if (ws_bytes < (encode_only ? l.enc_total : l.total))
    return set_error(DCKV_ECAPACITY, "workspace smaller than dckv_bytes() reports");
  return check_device(p);
}

int after_launch(const char *what) { return check_hip(hipGetLastError(), what); }


int encode_checks(const dckv_plan_t *plan, const uint16_t *rows, const int32_t *token_ids, int64_t T,
                  uint8_t *stream, uint64_t capacity, uint64_t *stream_bytes, int32_t *status, void *workspace,
                  uint64_t workspace_bytes, Geometry &g, Layout &l, bool encode_only = false) {
  int rc = common_checks(plan, T, workspace, workspace_bytes, status, g, l, encode_only);
  if (rc) return rc;
  if (T > 0 && (!rows || !aligned(rows, 16) || !token_ids || !aligned(token_ids, 4)))
    return set_error(DCKV_EINVAL, "rows must be 16-byte aligned, token_ids 4-byte aligned");
  if (!stream || !aligned(stream, 16) || !stream_bytes || !aligned(stream_bytes, 8))
    return set_error(DCKV_EINVAL, "stream must be 16-byte aligned and stream_bytes 8-byte aligned");
  if (capacity < g.fixed_bytes) return set_error(DCKV_ECAPACITY, "capacity below the stream's fixed part");
  return DCKV_OK;
}

int batch_error(int rc, int32_t i, const char *what) {
  char msg[160];
  std::snprintf(msg, sizeof msg, "%s: request %d: %s", what, (int)i, dckv_last_error());
  return set_error(rc, msg);
}

// Every stage runs over all n requests at once: one launch sequence per
// batch (up to kLaunchBatch requests per launch), so the tiles and groups of
// all requests share each launch and its load balance.
void encode_sequence(const EncodeArgs *a, int n) {
  launch_start_encode(a, n);
  launch_analysis_gemm(a, n);
  launch_encode_fixup(a, n);
  launch_rans_encode(a, n);
  launch_scan_header(a, n);
  launch_pack(a, n);
}

int decode_checks(const dckv_plan_t *plan, const uint8_t *stream, uint64_t stream_bytes, const int32_t *token_ids,
                  int64_t T, uint16_t *rows_out, int32_t *status, void *workspace, uint64_t workspace_bytes,
                  Geometry &g, Layout &l) {
  int rc = common_checks(plan, T, workspace, workspace_bytes, status, g, l);
  if (rc) return rc;
  if (T > 0 && (!rows_out || !aligned(rows_out, 16) || !token_ids || !aligned(token_ids, 4)))
    return set_error(DCKV_EINVAL, "rows_out must be 16-byte aligned, token_ids 4-byte aligned");
  if (!stream || !aligned(stream, 16)) return set_error(DCKV_EINVAL, "stream must be 16-byte aligned");
  if (stream_bytes < g.fixed_bytes) return set_error(DCKV_ECORRUPT, "stream shorter than its fixed part");
  return DCKV_OK;
}

void decode_sequence(const DecodeArgs *a, int n) {
  launch_parse(a, n, true);
  launch_rans_decode(a, n);
  launch_dequant(a, n);
  launch_w1_gemm(a, n);  // also RoPE on the kept rows
  launch_synthesis_gemm(a, n);
}

// Workspace slices of a batch: request i at offsets[i], each 256-byte aligned
// and as large as dckv_bytes() reports for it.
int batch_slices(const dckv_req *reqs, int32_t n, std::vector<uint64_t> &offsets, uint64_t &total) {
  offsets.assign((size_t)std::max(n, 0), 0);
  total = 0;
  for (int32_t i = 0; i < n; ++i) {
    uint64_t ws = 0;
    const int rc = dckv_bytes(reqs[i].plan, reqs[i].T, nullptr, &ws);
    if (rc) return batch_error(rc, i, "batch");
    offsets[i] = total;
    total += (ws + 255) & ~(uint64_t)255;
  }
  total = std::max<uint64_t>(total, 256);
  return DCKV_OK;
}

}  // namespace

extern "C" int dckv_encode(const dckv_plan_t *plan, const uint16_t *rows, const int32_t *token_ids, int64_t T,
                           uint8_t *stream, uint64_t capacity, uint64_t *stream_bytes, int32_t *status,
                           void *workspace, uint64_t workspace_bytes, void *hip_stream) {
  Geometry g;
  Layout l;
  int rc = encode_checks(plan, rows, token_ids, T, stream, capacity, stream_bytes, status, workspace,
                         workspace_bytes, g, l);
  if (rc) return rc;
  const EncodeArgs a{plan, g, l, static_cast<uint8_t *>(workspace), rows, token_ids, stream, capacity,
                     stream_bytes, status, static_cast<hipStream_t>(hip_stream)};
  encode_sequence(&a, 1);
  return after_launch("dckv_encode");
}

extern "C" int dckv_decode(const dckv_plan_t *plan, const uint8_t *stream, uint64_t stream_bytes,
                           const int32_t *token_ids, int64_t T, uint16_t *rows_out, int32_t *status,
                           void *workspace, uint64_t workspace_bytes, void *hip_stream) {
  Geometry g;
  Layout l;
  int rc = decode_checks(plan, stream, stream_bytes, token_ids, T, rows_out, status, workspace, workspace_bytes,
                         g, l);
  if (rc) return rc;
  const DecodeArgs a{plan, g, l, static_cast<uint8_t *>(workspace), stream, stream_bytes, token_ids,
                     rows_out, status, static_cast<hipStream_t>(hip_stream)};
  decode_sequence(&a, 1);
  return after_launch("dckv_decode");
}

extern "C" int dckv_decode_heads(const dckv_plan_t *plan, const uint8_t *stream, uint64_t stream_bytes,
                                 const int32_t *token_ids, int64_t T, uint16_t *const *kv_out, int32_t *status,
                                 void *workspace, uint64_t workspace_bytes, void *hip_stream) {
  Geometry g;
  Layout l;
  if (!kv_out) return set_error(DCKV_EINVAL, "decode_heads: null kv_out");
  KvHeads h;
  for (int i = 0; i < 12; ++i) {
    h.p[i] = kv_out[i];
    if (T > 0 && (!h.p[i] || !aligned(h.p[i], 16)))
      return set_error(DCKV_EINVAL, "decode_heads: every kv_out matrix must be a 16-byte aligned device pointer");
  }
  // rows_out is not used; pass a placeholder that satisfies the shared checks
  int rc = decode_checks(plan, stream, stream_bytes, token_ids, T, h.p[0], status, workspace, workspace_bytes, g, l);
  if (rc) return rc;
  DecodeArgs a{plan, g, l, static_cast<uint8_t *>(workspace), stream, stream_bytes, token_ids, nullptr, status,
               static_cast<hipStream_t>(hip_stream)};
  a.heads = &h;
  decode_sequence(&a, 1);
  return after_launch("dckv_decode_heads");
}

extern "C" int dckv_bytes_batch(const dckv_req *reqs, int32_t n, uint64_t *workspace_bytes) {
  if (n < 0 || (n > 0 && !reqs) || !workspace_bytes) return set_error(DCKV_EINVAL, "bytes_batch: bad argument");
  std::vector<uint64_t> off;
  uint64_t total = 0;
  const int rc = batch_slices(reqs, n, off, total);
  if (rc) return rc;
  *workspace_bytes = total;
  return DCKV_OK;
}

extern "C" int dckv_encode_batch(const dckv_req *reqs, int32_t n, void *workspace, uint64_t workspace_bytes,
                                 void *hip_stream) {
  if (n < 0 || (n > 0 && !reqs)) return set_error(DCKV_EINVAL, "encode_batch: bad argument");
  std::vector<uint64_t> off;
  uint64_t total = 0;
  int rc = batch_slices(reqs, n, off, total);
  if (rc) return rc;
  if (!workspace || workspace_bytes < total)
    return set_error(DCKV_ECAPACITY, "encode_batch: workspace smaller than dckv_bytes_batch() reports");
  std::vector<EncodeArgs> args;
  args.reserve(n);
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  for (int32_t i = 0; i < n; ++i) {
    const dckv_req &r = reqs[i];
    Geometry g;
    Layout l;
    rc = encode_checks(r.plan, r.rows, r.token_ids, r.T, r.stream, r.capacity, r.stream_bytes, r.status,
                       ws + off[i], total - off[i], g, l);
    if (rc) return batch_error(rc, i, "encode_batch");
    if (i > 0 && r.plan->device != reqs[0].plan->device)
      return batch_error(DCKV_EINVAL, i, "encode_batch: plans on different devices");
    args.push_back(EncodeArgs{r.plan, g, l, ws + off[i], r.rows, r.token_ids, r.stream, r.capacity, r.stream_bytes,
                              r.status, static_cast<hipStream_t>(hip_stream)});
  }
  if (n > 0) encode_sequence(args.data(), n);
  return after_launch("dckv_encode_batch");
}

extern "C" int dckv_decode_batch(const dckv_req *reqs, int32_t n, void *workspace, uint64_t workspace_bytes,
                                 void *hip_stream) {
  if (n < 0 || (n > 0 && !reqs)) return set_error(DCKV_EINVAL, "decode_batch: bad argument");
  std::vector<uint64_t> off;
  uint64_t total = 0;
  int rc = batch_slices(reqs, n, off, total);
  if (rc) return rc;
  if (!workspace || workspace_bytes < total)
    return set_error(DCKV_ECAPACITY, "decode_batch: workspace smaller than dckv_bytes_batch() reports");
  std::vector<DecodeArgs> args;
  args.reserve(n);
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  for (int32_t i = 0; i < n; ++i) {
    const dckv_req &r = reqs[i];
    Geometry g;
    Layout l;
    rc = decode_checks(r.plan, r.stream, r.capacity, r.token_ids, r.T, r.rows_out, r.status, ws + off[i],
                       total - off[i], g, l);
    if (rc) return batch_error(rc, i, "decode_batch");
    if (i > 0 && r.plan->device != reqs[0].plan->device)
      return batch_error(DCKV_EINVAL, i, "decode_batch: plans on different devices");
    args.push_back(DecodeArgs{r.plan, g, l, ws + off[i], r.stream, r.capacity, r.token_ids, r.rows_out, r.status,
                              static_cast<hipStream_t>(hip_stream)});
  }
  if (n > 0) decode_sequence(args.data(), n);
  return after_launch("dckv_decode_batch");
}

extern "C" int dckv_entropy_encode(const dckv_plan_t *plan, int64_t T, const uint8_t *sym, const uint32_t *esc,
                                   uint32_t n_esc, const uint16_t *rows, uint8_t *stream, uint64_t capacity,
                                   uint64_t *stream_bytes, int32_t *status, void *workspace,
                                   uint64_t workspace_bytes, void *hip_stream) {
  Geometry g;
  Layout l;
  int rc = common_checks(plan, T, workspace, workspace_bytes, status, g, l);
  if (rc) return rc;
  if (g.N > 0 && plan->C_a > 0 && !sym) return set_error(DCKV_EINVAL, "null symbols");
  if (n_esc > 0 && (!esc || !aligned(esc, 4))) return set_error(DCKV_EINVAL, "null or misaligned escapes");
  if ((int64_t)n_esc > g.esc_cap) return set_error(DCKV_ECAPACITY, "more escapes than the workspace holds");
  if (g.n_kept > 0 && (!rows || !aligned(rows, 16))) return set_error(DCKV_EINVAL, "rows must be 16-byte aligned");
  if (!stream || !aligned(stream, 16) || !stream_bytes || !aligned(stream_bytes, 8))
    return set_error(DCKV_EINVAL, "stream must be 16-byte aligned and stream_bytes 8-byte aligned");
  if (capacity < g.fixed_bytes) return set_error(DCKV_ECAPACITY, "capacity below the stream's fixed part");
  EncodeArgs a{plan, g, l, static_cast<uint8_t *>(workspace), rows, nullptr, stream, capacity,
               stream_bytes, status, static_cast<hipStream_t>(hip_stream)};
  launch_start_encode(&a, 1);
  launch_sym_to_tiled(a, sym);
  launch_load_esc(a, esc, n_esc);
  launch_rans_encode(&a, 1);
  launch_scan_header(&a, 1);
  launch_pack(&a, 1);
  return after_launch("dckv_entropy_encode");
}

extern "C" int dckv_entropy_decode(const dckv_plan_t *plan, const uint8_t *stream, uint64_t stream_bytes,
                                   int64_t T, uint8_t *sym_out, uint32_t *n_esc_out, int32_t *status,
                                   void *workspace, uint64_t workspace_bytes, void *hip_stream) {
  Geometry g;
  Layout l;
  int rc = common_checks(plan, T, workspace, workspace_bytes, status, g, l);
  if (rc) return rc;
  if (g.N > 0 && plan->C_a > 0 && !sym_out) return set_error(DCKV_EINVAL, "null sym_out");
  if (!stream || !aligned(stream, 16)) return set_error(DCKV_EINVAL, "stream must be 16-byte aligned");
  if (stream_bytes < g.fixed_bytes) return set_error(DCKV_ECORRUPT, "stream shorter than its fixed part");
  DecodeArgs a{plan, g, l, static_cast<uint8_t *>(workspace), stream, stream_bytes, nullptr, nullptr, status,
               static_cast<hipStream_t>(hip_stream)};
  launch_parse(&a, 1, false);
  launch_rans_decode(&a, 1);
  launch_sym_from_tiled(a, sym_out, n_esc_out);
  return after_launch("dckv_entropy_decode");
}

extern "C" int dckv_fit_bytes(int64_t n, uint64_t *workspace_bytes) {
  if (n < 2 || n > kMaxRows) return set_error(DCKV_EINVAL, "fit: n must be in [2, 2^18]");
  if (!workspace_bytes) return set_error(DCKV_EINVAL, "fit: null workspace_bytes");
  *workspace_bytes = fit_layout(n).total;
  return DCKV_OK;
}

extern "C" int dckv_fit(const dckv_params *p, const uint16_t *rows, const int32_t *token_ids, int64_t n, float ridge,
                        float *mean_head_out, uint16_t *mean_head_bf16_out, float *nbr_weight_out,
                        float *laplace_scale_out, int32_t *status, void *workspace, uint64_t workspace_bytes,
                        void *hip_stream) {
  if (!p) return set_error(DCKV_EINVAL, "fit: null params");
  if (p->n_layers != 6 || p->n_kv_heads != 2 || p->head_dim != kHeadDim || p->n_coef != kC || p->emb_dim != kEmb)
    return set_error(DCKV_EUNSUPPORTED,
                     "fit: the kernels support n_layers=6, n_kv_heads=2, head_dim=256, n_coef=2048, emb_dim=2048");
  if (!p->analysis || !p->embedding || p->vocab < 1) return set_error(DCKV_EINVAL, "fit: null analysis or embedding");
  uint64_t need = 0;
  int rc = dckv_fit_bytes(n, &need);
  if (rc) return rc;
  if (!rows || !aligned(rows, 16) || !token_ids || !aligned(token_ids, 4))
    return set_error(DCKV_EINVAL, "fit: rows must be 16-byte aligned, token_ids 4-byte aligned");
  if (!(ridge >= 0.0f) || !std::isfinite(ridge)) return set_error(DCKV_EINVAL, "fit: ridge must be finite and >= 0");
  if (!nbr_weight_out || !laplace_scale_out || !aligned(nbr_weight_out, 4) || !aligned(laplace_scale_out, 4))
    return set_error(DCKV_EINVAL, "fit: null or misaligned nbr_weight_out / laplace_scale_out");
  if ((mean_head_out && !aligned(mean_head_out, 4)) || (mean_head_bf16_out && !aligned(mean_head_bf16_out, 2)))
    return set_error(DCKV_EINVAL, "fit: misaligned mean head output");
  if (!status || !aligned(status, 4)) return set_error(DCKV_EINVAL, "fit: status must be a 4-byte aligned device word");
  if (!workspace || !aligned(workspace, 256)) return set_error(DCKV_EINVAL, "fit: workspace must be 256-byte aligned");
  if (workspace_bytes < need) return set_error(DCKV_ECAPACITY, "fit: workspace smaller than dckv_fit_bytes()");
  FitArgs a;
  a.l = fit_layout(n);
  a.ws = static_cast<uint8_t *>(workspace);
  a.rows = rows;
  a.A = p->analysis;
  a.E = p->embedding;
  a.tok = token_ids;
  a.n = n;
  a.vocab = p->vocab;
  a.ridge = ridge;
  a.H_out = mean_head_out;
  a.Hb_out = mean_head_bf16_out;
  a.a_out = nbr_weight_out;
  a.b_out = laplace_scale_out;
  a.status = status;
  a.s = static_cast<hipStream_t>(hip_stream);
  fit_sequence(a);
  return after_launch("dckv_fit");
}

extern "C" int dckv_rate_bytes(const dckv_plan_t *plan, int64_t T, uint64_t *workspace_bytes) {
  if (!plan) return set_error(DCKV_EINVAL, "rate: null plan");
  if (T < 0 || T > kMaxRows) return set_error(DCKV_EINVAL, "rate: T out of range (at most 2^18 positions)");
  if (!workspace_bytes) return set_error(DCKV_EINVAL, "rate: null workspace_bytes");
  *workspace_bytes = rate_layout(geometry(plan, T).N).total;
  return DCKV_OK;
}

extern "C" int dckv_rate_forward(const dckv_plan_t *plan, const uint16_t *rows, const int32_t *token_ids, int64_t T,
                                 const float *noise, float *bits_out, float *yhat_out, float *grad_y,
                                 float *grad_mean, float *grad_nbr, float *grad_scale, int32_t *status,
                                 void *workspace, uint64_t workspace_bytes, void *hip_stream) {
  uint64_t need = 0;
  int rc = dckv_rate_bytes(plan, T, &need);
  if (rc) return rc;
  if (plan->n_kv_heads != 2 || plan->head_dim != kHeadDim || plan->D != kD || plan->C != kC || plan->emb != kEmb)
    return set_error(DCKV_EUNSUPPORTED, "rate: the kernels support D=6144, n_coef=2048, emb_dim=2048");
  const int64_t N = geometry(plan, T).N;
  if (N > 0) {
    if (!rows || !aligned(rows, 16) || !token_ids || !aligned(token_ids, 4))
      return set_error(DCKV_EINVAL, "rate: rows must be 16-byte aligned, token_ids 4-byte aligned");
    const void *per_row[] = {noise, bits_out, yhat_out, grad_y, grad_mean};
    for (const void *q : per_row)
      if (!q || !aligned(q, 4)) return set_error(DCKV_EINVAL, "rate: null or misaligned per-row array");
  }
  if (!grad_nbr || !grad_scale || !aligned(grad_nbr, 4) || !aligned(grad_scale, 4))
    return set_error(DCKV_EINVAL, "rate: null or misaligned grad_nbr / grad_scale");
  if (!status || !aligned(status, 4)) return set_error(DCKV_EINVAL, "rate: status must be a 4-byte aligned device word");
  if (!workspace || !aligned(workspace, 256)) return set_error(DCKV_EINVAL, "rate: workspace must be 256-byte aligned");
  if (workspace_bytes < need) return set_error(DCKV_ECAPACITY, "rate: workspace smaller than dckv_rate_bytes()");
  rc = check_device(plan);
  if (rc) return rc;
  RateArgs a;
  a.p = plan;
  a.l = rate_layout(N);
  a.ws = static_cast<uint8_t *>(workspace);
  a.rows = rows;
  a.tok = token_ids;
  a.noise = noise;
  a.N = N;
  a.bits = bits_out;
  a.yhat = yhat_out;
  a.grad_y = grad_y;
  a.grad_mean = grad_mean;
  a.grad_nbr = grad_nbr;
  a.grad_scale = grad_scale;
  a.status = status;
  a.s = static_cast<hipStream_t>(hip_stream);
  rate_sequence(a);
  return after_launch("dckv_rate_forward");
}

extern "C" int dckv_rate_backward_bytes(const dckv_plan_t *plan, int64_t T, uint64_t *workspace_bytes) {
  if (!plan) return set_error(DCKV_EINVAL, "rate backward: null plan");
  if (T < 0 || T > kMaxRows) return set_error(DCKV_EINVAL, "rate backward: T out of range (at most 2^18 positions)");
  if (!workspace_bytes) return set_error(DCKV_EINVAL, "rate backward: null workspace_bytes");
  *workspace_bytes = rate_bwd_layout(geometry(plan, T).N).total;
  return DCKV_OK;
}

extern "C" int dckv_rate_backward(const dckv_plan_t *plan, const uint16_t *rows, const int32_t *token_ids,
                                  int64_t T, const float *grad_y, const float *grad_mean, float *grad_analysis,
                                  float *grad_mean_head, int32_t *status, void *workspace, uint64_t workspace_bytes,
                                  void *hip_stream) {
  uint64_t need = 0;
  int rc = dckv_rate_backward_bytes(plan, T, &need);
  if (rc) return rc;
  if (plan->D != kD || plan->C != kC || plan->emb != kEmb)
    return set_error(DCKV_EUNSUPPORTED, "rate backward: the kernels support D=6144, n_coef=2048, emb_dim=2048");
  const int64_t N = geometry(plan, T).N;
  if (N > 0) {
    if (!rows || !aligned(rows, 16) || !token_ids || !aligned(token_ids, 4))
      return set_error(DCKV_EINVAL, "rate backward: rows must be 16-byte aligned, token_ids 4-byte aligned");
    if (!grad_y || !grad_mean || !aligned(grad_y, 16) || !aligned(grad_mean, 16))
      return set_error(DCKV_EINVAL, "rate backward: grad_y / grad_mean must be 16-byte aligned");
  }
  if (!grad_analysis || !grad_mean_head || !aligned(grad_analysis, 4) || !aligned(grad_mean_head, 4))
    return set_error(DCKV_EINVAL, "rate backward: null or misaligned grad_analysis / grad_mean_head");
  if (!status || !aligned(status, 4))
    return set_error(DCKV_EINVAL, "rate backward: status must be a 4-byte aligned device word");
  if (!workspace || !aligned(workspace, 256))
    return set_error(DCKV_EINVAL, "rate backward: workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return set_error(DCKV_ECAPACITY, "rate backward: workspace smaller than dckv_rate_backward_bytes()");
  rc = check_device(plan);
  if (rc) return rc;
  RateBwdArgs a;
  a.p = plan;
  a.l = rate_bwd_layout(N);
  a.ws = static_cast<uint8_t *>(workspace);
  a.rows = rows;
  a.tok = token_ids;
  a.grad_y = grad_y;
  a.grad_mean = grad_mean;
  a.N = N;
  a.grad_A = grad_analysis;
  a.grad_H = grad_mean_head;
  a.status = status;
  a.s = static_cast<hipStream_t>(hip_stream);
  rate_bwd_sequence(a);
  return after_launch("dckv_rate_backward");
}

extern "C" int dckv_unrope(const dckv_plan_t *plan, const uint16_t *rows_in, int64_t T, uint16_t *rows_out,
                           void *hip_stream) {
  if (!plan) return set_error(DCKV_EINVAL, "unrope: null plan");
  if (T < 0 || T > 0x7FFFFFFF) return set_error(DCKV_EINVAL, "unrope: T out of range");
  if (T > 0 && (!rows_in || !rows_out || !aligned(rows_in, 4) || !aligned(rows_out, 4)))
    return set_error(DCKV_EINVAL, "unrope: rows must be 4-byte aligned device pointers");
  int rc = check_device(plan);
  if (rc) return rc;
  launch_unrope(plan, rows_in, rows_out, T, static_cast<hipStream_t>(hip_stream));
  return after_launch("dckv_unrope");
}

// ---------------------------------------------------------------------------
// Encode without any allocation: the workspace is a file-scope device array.
// Every device the library runs on holds its own copy of the array until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it only names a stand-in): the device address of each device's copy
// comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is used.
// ---------------------------------------------------------------------------
namespace {
constexpr uint64_t kNoAllocScratchBytes = 72ull << 20;
constexpr int kNoAllocMaxDevices = 64;
}  // namespace

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
std::mutex g_scratch_mu;
void *g_scratch_dev[kNoAllocMaxDevices] = {};

// The calling thread's current device must be `dev`.
int scratch_address(int dev, void **out) {
  if (dev < 0 || dev >= kNoAllocMaxDevices) return set_error(DCKV_EUNSUPPORTED, "encode_noalloc: device index too large");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return check_hip(e != hipSuccess ? e : hipErrorInvalidSymbol, "encode_noalloc: scratch address");
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return DCKV_OK;
}
}  // namespace

extern "C" int dckv_encode_noalloc(const dckv_plan_t *plan, const uint16_t *rows, const int32_t *token_ids, int64_t T,
                                   uint8_t *stream, uint64_t capacity, uint64_t *stream_bytes, int32_t *status,
                                   void *hip_stream) {
  if (!plan) return set_error(DCKV_EINVAL, "encode_noalloc: null plan");
  if (T < 0 || T > kMaxRows) return set_error(DCKV_EINVAL, "encode_noalloc: T out of range");
  int rc = check_device(plan);
  if (rc) return rc;
  const Geometry g0 = geometry(plan, T);
  const Layout l0 = layout(plan, g0);
  if (l0.enc_total > kNoAllocScratchBytes) {
    char msg[200];
    std::snprintf(msg, sizeof msg,
                  "encode_noalloc: a %lld-position request needs %llu bytes of scratch; the library holds %llu "
                  "(every plan fits up to 8,192 positions); use dckv_encode with a workspace",
                  (long long)T, (unsigned long long)l0.enc_total, (unsigned long long)kNoAllocScratchBytes);
    return set_error(DCKV_ECAPACITY, msg);
  }
  void *ws = nullptr;
  rc = scratch_address(plan->device, &ws);
  if (rc) return rc;
  Geometry g;
  Layout l;
  rc = encode_checks(plan, rows, token_ids, T, stream, capacity, stream_bytes, status, ws, kNoAllocScratchBytes, g,
                     l, /*encode_only=*/true);
  if (rc) return rc;
  const EncodeArgs a{plan, g, l, static_cast<uint8_t *>(ws), rows, token_ids, stream, capacity, stream_bytes,
                     status, static_cast<hipStream_t>(hip_stream)};
  encode_sequence(&a, 1);
  return after_launch("dckv_encode_noalloc");
}

// ---------------------------------------------------------------------------
// Encode from a post-RoPE cache: the key heads are rotated back into a copy in
// the workspace (fp64, one bf16 rounding, as dckv_unrope), then the usual
// encode reads its key k-tiles and kept-row keys from that copy and its value
// k-tiles from the caller's rows.
// ---------------------------------------------------------------------------
namespace {
uint64_t postrope_keys_offset(const Layout &l) { return (l.enc_total + 255) & ~(uint64_t)255; }
}  // namespace

extern "C" int dckv_bytes_postrope(const dckv_plan_t *plan, int64_t T, uint64_t *workspace_bytes) {
  uint64_t ws = 0;
  const int rc = dckv_bytes(plan, T, nullptr, &ws);
  if (rc) return rc;
  if (!workspace_bytes) return set_error(DCKV_EINVAL, "bytes_postrope: null workspace_bytes");
  const Layout l = layout(plan, geometry(plan, T));
  *workspace_bytes = postrope_keys_offset(l) + (uint64_t)std::max<int64_t>(T, 1) * kKeyCols * 2;
  return DCKV_OK;
}

extern "C" int dckv_encode_postrope(const dckv_plan_t *plan, const uint16_t *rows, const int32_t *token_ids,
                                    int64_t T, uint8_t *stream, uint64_t capacity, uint64_t *stream_bytes,
                                    int32_t *status, void *workspace, uint64_t workspace_bytes, void *hip_stream) {
  uint64_t need = 0;
  int rc = dckv_bytes_postrope(plan, T, &need);
  if (rc) return rc;
  if (workspace_bytes < need)
    return set_error(DCKV_ECAPACITY, "encode_postrope: workspace smaller than dckv_bytes_postrope() reports");
  Geometry g;
  Layout l;
  rc = encode_checks(plan, rows, token_ids, T, stream, capacity, stream_bytes, status, workspace, workspace_bytes, g,
                     l, /*encode_only=*/true);
  if (rc) return rc;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  uint16_t *keys = reinterpret_cast<uint16_t *>(ws + postrope_keys_offset(l));
  const hipStream_t s = static_cast<hipStream_t>(hip_stream);
  launch_unrope_keys(plan, rows, keys, T, s);
  EncodeArgs a{plan, g, l, ws, rows, token_ids, stream, capacity, stream_bytes, status, s};
  a.keys = keys;
  encode_sequence(&a, 1);
  return after_launch("dckv_encode_postrope");
}

// ---------------------------------------------------------------------------
// A paged attention cache on either side of the codec: encode gathers the
// request's rows from the pools (rotating the keys back when they carry RoPE)
// into the workspace and encodes them; decode decodes into the workspace and
// scatters the rows into the pools.  The block table is checked on the device
// first: an entry outside [0, n_blocks) makes the call's status EINVAL and
// nothing is read from (encode) or written to (decode) the pools.
// ---------------------------------------------------------------------------
namespace {
// workspace of a paged call: the codec's workspace, the rows, one status word
uint64_t paged_rows_offset(const Layout &l) { return (l.total + 255) & ~(uint64_t)255; }
uint64_t paged_pre_offset(const Layout &l, int64_t T) {
  return paged_rows_offset(l) + (((uint64_t)std::max<int64_t>(T, 1) * kD * 2 + 255) & ~(uint64_t)255);
}

int paged_from(const dckv_paged_kv *c, int64_t T, PagedKV &kv, const char *what) {
  char msg[160];
  if (!c) {
    std::snprintf(msg, sizeof msg, "%s: null cache", what);
    return set_error(DCKV_EINVAL, msg);
  }
  if (c->block_size < 1 || c->n_blocks < 1 || (T > 0 && !c->block_table) || !aligned(c->block_table, 4)) {
    std::snprintf(msg, sizeof msg, "%s: block_size and n_blocks must be >= 1 and block_table a device int32 array",
                  what);
    return set_error(DCKV_EINVAL, msg);
  }
  for (int i = 0; i < 12; ++i) {
    kv.p[i] = c->kv[i];
    if (T > 0 && (!kv.p[i] || !aligned(kv.p[i], 16))) {
      std::snprintf(msg, sizeof msg, "%s: every pool must be a 16-byte aligned device pointer", what);
      return set_error(DCKV_EINVAL, msg);
    }
  }
  kv.table = c->block_table;
  kv.bs = c->block_size;
  kv.n_blocks = c->n_blocks;
  return DCKV_OK;
}
}  // namespace

extern "C" int dckv_bytes_paged(const dckv_plan_t *plan, int64_t T, uint64_t *workspace_bytes) {
  uint64_t ws = 0;
  const int rc = dckv_bytes(plan, T, nullptr, &ws);
  if (rc) return rc;
  if (!workspace_bytes) return set_error(DCKV_EINVAL, "bytes_paged: null workspace_bytes");
  const Layout l = layout(plan, geometry(plan, T));
  *workspace_bytes = paged_pre_offset(l, T) + 256;
  return DCKV_OK;
}

extern "C" int dckv_encode_paged(const dckv_plan_t *plan, const dckv_paged_kv *cache, int32_t post_rope,
                                 const int32_t *token_ids, int64_t T, uint8_t *stream, uint64_t capacity,
                                 uint64_t *stream_bytes, int32_t *status, void *workspace, uint64_t workspace_bytes,
                                 void *hip_stream) {
  uint64_t need = 0;
  int rc = dckv_bytes_paged(plan, T, &need);
  if (rc) return rc;
  if (workspace_bytes < need)
    return set_error(DCKV_ECAPACITY, "encode_paged: workspace smaller than dckv_bytes_paged() reports");
  PagedKV kv;
  rc = paged_from(cache, T, kv, "encode_paged");
  if (rc) return rc;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  const Layout l0 = layout(plan, geometry(plan, T));
  uint16_t *rows = reinterpret_cast<uint16_t *>(ws + paged_rows_offset(l0));
  int32_t *pre = reinterpret_cast<int32_t *>(ws + paged_pre_offset(l0, T));
  Geometry g;
  Layout l;
  rc = encode_checks(plan, rows, token_ids, T, stream, capacity, stream_bytes, status, workspace, workspace_bytes, g,
                     l);
  if (rc) return rc;
  const hipStream_t s = static_cast<hipStream_t>(hip_stream);
  launch_paged_check(kv, T, pre, true, s);
  launch_paged_gather(plan, kv, post_rope != 0, T, rows, pre, s);
  EncodeArgs a{plan, g, l, ws, rows, token_ids, stream, capacity, stream_bytes, status, s};
  a.pre = pre;
  encode_sequence(&a, 1);
  return after_launch("dckv_encode_paged");
}

extern "C" int dckv_decode_paged(const dckv_plan_t *plan, const uint8_t *stream, uint64_t stream_bytes,
                                 const int32_t *token_ids, int64_t T, const dckv_paged_kv *cache, int32_t *status,
                                 void *workspace, uint64_t workspace_bytes, void *hip_stream) {
  uint64_t need = 0;
  int rc = dckv_bytes_paged(plan, T, &need);
  if (rc) return rc;
  if (workspace_bytes < need)
    return set_error(DCKV_ECAPACITY, "decode_paged: workspace smaller than dckv_bytes_paged() reports");
  PagedKV kv;
  rc = paged_from(cache, T, kv, "decode_paged");
  if (rc) return rc;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  const Layout l0 = layout(plan, geometry(plan, T));
  uint16_t *rows = reinterpret_cast<uint16_t *>(ws + paged_rows_offset(l0));
  Geometry g;
  Layout l;
  rc = decode_checks(plan, stream, stream_bytes, token_ids, T, rows, status, workspace, workspace_bytes, g, l);
  if (rc) return rc;
  const hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const DecodeArgs a{plan, g, l, ws, stream, stream_bytes, token_ids, rows, status, s};
  decode_sequence(&a, 1);
  // after the decode: its parse clears the status first
  launch_paged_check(kv, T, status, false, s);
  launch_paged_scatter(kv, T, rows, status, s);
  return after_launch("dckv_decode_paged");
}
