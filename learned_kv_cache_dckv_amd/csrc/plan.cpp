// Host runtime of the DCKV codec library: rate plan (steps, dropped
// components, integer Laplace tables, CRC), device upload, request geometry,
// workspace layout, error reporting and kernel timing.
//
// The plan follows the DCKV digest page ("DCKV: Learned Transform Coding of
// the Prompt KV Cache in Hybrid Language Models"), "How it works": the
// Transform bullet (per-component steps, components under 0.05 steps are
// dropped) and the Coding bullet (rANS under Laplace distributions, codes
// beyond +-127 escaped).  The table construction is the discretised Laplace
// of scale b_c/step_c over the 255 codes -127..127, renormalised, at 15-bit
// precision; it depends on no float prediction, so encoder and decoder always
// select identical tables (the concern raised in the page's "Limits").
// Table arithmetic must round exactly as written: no contraction into FMA.
#pragma clang fp contract(off)

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "dckv_internal.h"

using namespace dckv;

// ---------------------------------------------------------------------------
// errors
// ---------------------------------------------------------------------------
static thread_local std::string g_last_error;

int dckv::set_error(int code, const std::string &msg) {
  g_last_error = msg;
  return code;
}

int dckv::check_hip(hipError_t e, const char *what) {
  if (e == hipSuccess) return DCKV_OK;
  return set_error(DCKV_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

extern "C" const char *dckv_last_error(void) { return g_last_error.c_str(); }

// ---------------------------------------------------------------------------
// CRC-32, reflected polynomial 0xEDB88320 (the zlib/PNG CRC), table driven
// ---------------------------------------------------------------------------
namespace {
struct Crc32 {
  uint32_t t[256];
  Crc32() {
    for (uint32_t i = 0; i < 256; ++i) {
      uint32_t c = i;
      for (int k = 0; k < 8; ++k) c = (c & 1u) ? (c >> 1) ^ 0xEDB88320u : (c >> 1);
      t[i] = c;
    }
  }
  uint32_t update(uint32_t crc, const uint8_t *p, size_t n) const {
    crc = ~crc;
    for (size_t i = 0; i < n; ++i) crc = t[(crc ^ p[i]) & 0xFFu] ^ (crc >> 8);
    return ~crc;
  }
};
const Crc32 &crc_tab() {
  static Crc32 c;
  return c;
}

// Integer table of one component with Laplace scale s (in steps).
void laplace_table(double s, uint16_t *f_out) {
  double p[kNSym];
  for (int i = 0; i < kNSym; ++i) {
    const int k = i - 127;
    if (k == 0) {
      p[i] = 1.0 - std::exp(-0.5 / s);
    } else {
      const double ak = (double)(k < 0 ? -k : k);
      p[i] = 0.5 * std::exp(-(ak - 0.5) / s) - 0.5 * std::exp(-(ak + 0.5) / s);
    }
  }
  double total = 0.0;
  for (int i = 0; i < kNSym; ++i) total = total + p[i];  // index order
  int64_t sum = 0;
  int64_t f[kNSym];
  for (int i = 0; i < kNSym; ++i) {
    f[i] = 1 + (int64_t)std::floor((p[i] / total) * (double)(kM - kNSym));
    sum += f[i];
  }
  f[127] += (int64_t)kM - sum;
  for (int i = 0; i < kNSym; ++i) f_out[i] = (uint16_t)f[i];
}

struct HostTables {
  std::vector<float> step;
  std::vector<uint8_t> active;
  std::vector<int32_t> act;
  std::vector<uint16_t> freq;
  uint32_t crc = 0;
};

int build_tables(const float *base_step, const float *laplace_scale, int32_t n, float g, HostTables &h) {
  if (n < 1 || !base_step || !laplace_scale) return set_error(DCKV_EINVAL, "plan: bad vectors");
  if (!(g > 0.0f) || !std::isfinite(g)) return set_error(DCKV_EINVAL, "plan: step_scale must be finite and > 0");
  h.step.resize(n);
  h.active.resize(n);
  h.act.clear();
  for (int c = 0; c < n; ++c) {
    if (!(base_step[c] > 0.0f) || !std::isfinite(base_step[c]) || !(laplace_scale[c] >= 0.0f) ||
        !std::isfinite(laplace_scale[c]))
      return set_error(DCKV_EINVAL, "plan: base_step must be > 0 and laplace_scale >= 0, finite");
    volatile float st = g * base_step[c];  // one IEEE float32 product
    h.step[c] = st;
    if (!(h.step[c] > 0.0f) || !std::isfinite(h.step[c]))
      return set_error(DCKV_EINVAL, "plan: step underflows or overflows");
    const double s = (double)laplace_scale[c] / (double)h.step[c];
    h.active[c] = s >= 0.05 ? 1 : 0;
    if (h.active[c]) h.act.push_back(c);
  }
  const int Ca = (int)h.act.size();
  h.freq.assign((size_t)Ca * kNSym, 0);
  for (int r = 0; r < Ca; ++r) {
    const int c = h.act[r];
    laplace_table((double)laplace_scale[c] / (double)h.step[c], &h.freq[(size_t)r * kNSym]);
  }
  // CRC over step (fp32 LE), active flags (u8), active frequencies (u16 LE)
  uint32_t crc = 0;
  crc = crc_tab().update(crc, reinterpret_cast<const uint8_t *>(h.step.data()), h.step.size() * 4);
  crc = crc_tab().update(crc, h.active.data(), h.active.size());
  crc = crc_tab().update(crc, reinterpret_cast<const uint8_t *>(h.freq.data()), h.freq.size() * 2);
  h.crc = crc;
  return DCKV_OK;
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }
}  // namespace

extern "C" int dckv_plan_tables(const float *base_step, const float *laplace_scale, int32_t n_coef,
                                float step_scale, float *step_out, uint8_t *active_out,
                                uint16_t *freq_out, int32_t *c_active, uint32_t *crc) {
  HostTables h;
  int rc = build_tables(base_step, laplace_scale, n_coef, step_scale, h);
  if (rc) return rc;
  if (step_out) std::memcpy(step_out, h.step.data(), h.step.size() * 4);
  if (active_out) std::memcpy(active_out, h.active.data(), h.active.size());
  if (freq_out) std::memcpy(freq_out, h.freq.data(), h.freq.size() * 2);
  if (c_active) *c_active = (int32_t)h.act.size();
  if (crc) *crc = h.crc;
  return DCKV_OK;
}

// ---------------------------------------------------------------------------
// shared embedding-mean tables
// ---------------------------------------------------------------------------
namespace {
struct MtKey {
  int device;
  const void *E, *H;
  int vocab;
  std::vector<int32_t> perm;
  bool operator<(const MtKey &o) const {
    if (device != o.device) return device < o.device;
    if (E != o.E) return E < o.E;
    if (H != o.H) return H < o.H;
    if (vocab != o.vocab) return vocab < o.vocab;
    return perm < o.perm;
  }
};
struct MtEntry {
  float *ptr;
  int users;
};
struct MtState {
  std::mutex mu;
  std::map<MtKey, MtEntry> tables;
};
MtState &mt_state() {
  static MtState s;
  return s;
}
MtKey mt_key(const dckv_plan_t *pl) { return MtKey{pl->device, pl->E, pl->H, pl->vocab, pl->mt_perm}; }

// Sets pl->mtab: an existing table of the same key (one more user), or a new
// one built by one GEMM (synchronous).  The lock is held while a table is
// built, so two plans never build the same table.
int acquire_mean_table(dckv_plan_t *pl, const std::vector<int32_t> &perm) {
  pl->mt_perm = perm;
  MtState &st = mt_state();
  std::lock_guard<std::mutex> lk(st.mu);
  const MtKey key = mt_key(pl);
  auto it = st.tables.find(key);
  if (it != st.tables.end()) {
    it->second.users += 1;
    pl->mtab = it->second.ptr;
    return DCKV_OK;
  }
  void *mtab = nullptr;
  if (hipMalloc(&mtab, (size_t)pl->vocab * pl->C * 4) != hipSuccess)
    return set_error(DCKV_ENOMEM, "plan: hipMalloc of the embedding-mean table failed");
  pl->mtab = static_cast<float *>(mtab);
  const int rc = build_mean_table(pl);
  if (rc) {
    (void)hipFree(mtab);
    pl->mtab = nullptr;
    return rc;
  }
  st.tables.emplace(key, MtEntry{pl->mtab, 1});
  return DCKV_OK;
}

// One user fewer; the last one frees the table (the plan's device is current).
int release_mean_table(dckv_plan_t *pl) {
  MtState &st = mt_state();
  std::lock_guard<std::mutex> lk(st.mu);
  auto it = st.tables.find(mt_key(pl));
  if (it == st.tables.end()) return set_error(DCKV_EINVAL, "plan_free: mean table not registered");
  if (--it->second.users > 0) return DCKV_OK;
  const int rc = check_hip(hipFree(it->second.ptr), "plan_free");
  st.tables.erase(it);
  return rc;
}
}  // namespace

extern "C" int dckv_plan(const dckv_params *p, float step_scale, dckv_plan_t **out) {
  if (!p || !out) return set_error(DCKV_EINVAL, "plan: null argument");
  *out = nullptr;
  if (p->n_layers != 6 || p->n_kv_heads != 2 || p->head_dim != kHeadDim || p->n_coef != kC ||
      p->n_hidden != kHid || p->emb_dim != kEmb)
    return set_error(DCKV_EUNSUPPORTED,
                     "plan: the kernels support n_layers=6, n_kv_heads=2, head_dim=256, n_coef=2048, "
                     "n_hidden=256, emb_dim=2048");
  if (p->vocab > kMaxVocab)
    return set_error(DCKV_EUNSUPPORTED, "plan: vocab above 2^19 - 1 (the mean table is addressed with 32-bit offsets)");
  if (p->vocab < 1 || p->keep_head < 0 || p->keep_tail < 0 || !(p->rope_theta > 0.0f) ||
      !std::isfinite(p->rope_theta))
    return set_error(DCKV_EINVAL, "plan: bad vocab, keep sizes or rope_theta");
  if (!p->analysis || !p->synthesis || !p->embedding || !p->mean_head || !p->nbr_weight)
    return set_error(DCKV_EINVAL, "plan: null parameter pointer");
  if (!p->w1 != !p->w2) return set_error(DCKV_EINVAL, "plan: w1 and w2 are both given or both null");
  for (int c = 0; c < p->n_coef; ++c)
    if (!std::isfinite(p->nbr_weight[c])) return set_error(DCKV_EINVAL, "plan: non-finite nbr_weight");
  HostTables h;
  int rc = build_tables(p->base_step, p->laplace_scale, p->n_coef, step_scale, h);
  if (rc) return rc;

  dckv_plan_t *pl = new dckv_plan_t();
  pl->n_layers = p->n_layers;
  pl->n_kv_heads = p->n_kv_heads;
  pl->head_dim = p->head_dim;
  pl->D = p->n_layers * 2 * p->n_kv_heads * p->head_dim;
  pl->C = p->n_coef;
  pl->hidden = p->n_hidden;
  pl->emb = p->emb_dim;
  pl->vocab = p->vocab;
  pl->keep_head = p->keep_head;
  pl->keep_tail = p->keep_tail;
  pl->rope_theta = p->rope_theta;
  pl->step_scale = step_scale;
  pl->C_a = (int)h.act.size();
  pl->G = (pl->C_a + kLanes - 1) / kLanes;
  pl->crc = h.crc;
  pl->step = h.step;
  pl->active = h.active;
  pl->freq = h.freq;
  pl->A = p->analysis;
  pl->S = p->synthesis;
  pl->W1 = p->w1;
  pl->W2 = p->w2;
  pl->E = p->embedding;
  pl->H = p->mean_head;
  if (hipGetDevice(&pl->device) != hipSuccess) {
    delete pl;
    return set_error(DCKV_EHIP, "plan: no HIP device");
  }

  // host images of the device arrays
  const int C = pl->C, Ca = pl->C_a;
  const int Ca_pad = (int)round_up(std::max(Ca, 1), kBN);
  std::vector<int32_t> rank(C, -1), act(Ca_pad, 0);
  for (int r = 0; r < Ca; ++r) {
    rank[h.act[r]] = r;
    act[r] = h.act[r];
  }
  for (int r = Ca; r < Ca_pad; ++r) act[r] = Ca > 0 ? h.act[Ca - 1] : 0;
  // mean-table columns: the active components in rank order, then the
  // dropped ones in ascending order
  std::vector<int32_t> perm(C), colpos(C);
  {
    int i = 0;
    for (int r = 0; r < Ca; ++r) perm[i++] = h.act[r];
    for (int c = 0; c < C; ++c)
      if (rank[c] < 0) perm[i++] = c;
    for (int k = 0; k < C; ++k) colpos[perm[k]] = k;
  }
  std::vector<uint32_t> tab((size_t)std::max(Ca, 1) * 256, 0);
  std::vector<float> rcp((size_t)std::max(Ca, 1) * 256, 0.f);
  std::vector<uint32_t> bucket((size_t)std::max(Ca, 1) * kBuckets, 0);
  for (int r = 0; r < Ca; ++r) {
    uint32_t cum = 0;
    const uint16_t *f = &h.freq[(size_t)r * kNSym];
    std::vector<uint32_t> cumv(kNSym + 1, 0);
    for (int s = 0; s < kNSym; ++s) {
      tab[(size_t)r * 256 + s] = (uint32_t)f[s] | (cum << 16);
      cumv[s] = cum;
      cum += f[s];
    }
    cumv[kNSym] = cum;
    // entry 255 (escape) codes as the identity in the encoder: f = 2^15, cum 0
    tab[(size_t)r * 256 + 255] = kM;
    // the encoder's reciprocal of f, scaled down by (1 - 2^-21) before its
    // rounding to fp32: fp32(x) * rcp then never exceeds x / f and stays above
    // x / f - 1 for x < 2^32, so the quotient needs one upward correction at most
    for (int s = 0; s < 256; ++s) {
      const uint32_t fs = tab[(size_t)r * 256 + s] & 0xFFFFu;
      rcp[(size_t)r * 256 + s] = (float)((1.0 / (double)fs) * (1.0 - std::ldexp(1.0, -21)));
    }
    // decoder buckets of 2^kBucketShift slots: lo = symbol of the bucket's
    // first slot; split = the slot where symbol lo + 1 starts when the bucket
    // holds exactly two symbols (so a slot's symbol is lo + (slot >= split)),
    // kSplitPure (no slot reaches it) when it holds one, kSplitSearch when it
    // holds three or more
    int s = 0;
    for (int b = 0; b < kBuckets; ++b) {
      const uint32_t first = (uint32_t)b << kBucketShift, last = first + (1u << kBucketShift) - 1u;
      while (cumv[s + 1] <= first) ++s;
      int e = s;
      while (cumv[e + 1] <= last) ++e;
      uint32_t split;
      if (e == s) split = kSplitPure;
      else if (e == s + 1) split = cumv[s + 1];
      else split = kSplitSearch;
      bucket[(size_t)r * kBuckets + b] = (uint32_t)s | (split << 16);
    }
  }
  // quantiser constants of each rank: step, 1 / step (0 past C_a), neighbour weight
  std::vector<float> qcol((size_t)Ca_pad * 4, 0.f);
  for (int r = 0; r < Ca_pad; ++r) {
    const int c = act[r];
    qcol[4 * r] = h.step[c];
    qcol[4 * r + 1] = r < Ca ? 1.0f / h.step[c] : 0.f;
    qcol[4 * r + 2] = p->nbr_weight[c];
  }
  std::vector<double> omega(kHalf);
  for (int i = 0; i < kHalf; ++i) omega[i] = std::pow((double)pl->rope_theta, -(double)i / (double)kHalf);

  // one device block
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const size_t o_step = take(C * 4), o_nbr = take(C * 4), o_rank = take(C * 4), o_act = take(Ca_pad * 4);
  const size_t o_perm = take(C * 4), o_colpos = take(C * 4), o_qcol = take(qcol.size() * 4), o_scale = take(C * 4);
  const size_t o_tab = take(tab.size() * 4), o_rcp = take(rcp.size() * 4), o_bucket = take(bucket.size() * 4);
  const size_t o_omega = take(kHalf * 8);
  void *blk = nullptr;
  if (hipMalloc(&blk, off) != hipSuccess) {
    delete pl;
    return set_error(DCKV_ENOMEM, "plan: hipMalloc of the device tables failed");
  }
  std::vector<uint8_t> img(off, 0);
  std::memcpy(&img[o_step], h.step.data(), C * 4);
  std::memcpy(&img[o_nbr], p->nbr_weight, C * 4);
  std::memcpy(&img[o_rank], rank.data(), C * 4);
  std::memcpy(&img[o_act], act.data(), Ca_pad * 4);
  std::memcpy(&img[o_perm], perm.data(), C * 4);
  std::memcpy(&img[o_colpos], colpos.data(), C * 4);
  std::memcpy(&img[o_qcol], qcol.data(), qcol.size() * 4);
  std::memcpy(&img[o_scale], p->laplace_scale, C * 4);
  std::memcpy(&img[o_tab], tab.data(), tab.size() * 4);
  std::memcpy(&img[o_rcp], rcp.data(), rcp.size() * 4);
  std::memcpy(&img[o_bucket], bucket.data(), bucket.size() * 4);
  std::memcpy(&img[o_omega], omega.data(), kHalf * 8);
  if (hipMemcpy(blk, img.data(), off, hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(blk);
    delete pl;
    return set_error(DCKV_EHIP, "plan: upload of the device tables failed");
  }
  uint8_t *b = static_cast<uint8_t *>(blk);
  pl->dev_block = blk;
  pl->dev.step = reinterpret_cast<float *>(b + o_step);
  pl->dev.nbr = reinterpret_cast<float *>(b + o_nbr);
  pl->dev.rank = reinterpret_cast<int32_t *>(b + o_rank);
  pl->dev.act = reinterpret_cast<int32_t *>(b + o_act);
  pl->dev.perm = reinterpret_cast<int32_t *>(b + o_perm);
  pl->dev.colpos = reinterpret_cast<int32_t *>(b + o_colpos);
  pl->dev.qcol = reinterpret_cast<float *>(b + o_qcol);
  pl->dev.scale = reinterpret_cast<float *>(b + o_scale);
  pl->dev.tab = reinterpret_cast<uint32_t *>(b + o_tab);
  pl->dev.rcp = reinterpret_cast<float *>(b + o_rcp);
  pl->dev.bucket = reinterpret_cast<uint32_t *>(b + o_bucket);
  pl->dev.omega = reinterpret_cast<double *>(b + o_omega);
  pl->dev_bytes = off;
  // the embedding-mean table: H E[v] for every token id, shared by the plans
  // that have the same device, embedding, mean head and column order
  rc = acquire_mean_table(pl, perm);
  if (rc) {
    (void)hipFree(blk);
    delete pl;
    return rc;
  }
  *out = pl;
  return DCKV_OK;
}

extern "C" int dckv_plan_free(dckv_plan_t *plan) {
  if (!plan) return DCKV_OK;
  int rc = DCKV_OK;
  if (plan->dev_block) {
    int cur = 0;
    (void)hipGetDevice(&cur);
    (void)hipSetDevice(plan->device);
    rc = check_hip(hipFree(plan->dev_block), "plan_free");
    if (plan->mtab) {
      const int rc2 = release_mean_table(plan);
      if (rc == DCKV_OK) rc = rc2;
    }
    (void)hipSetDevice(cur);
  }
  delete plan;
  return rc;
}

extern "C" int dckv_plan_memory(const dckv_plan_t *plan, uint64_t *table_bytes, uint64_t *mean_table_bytes,
                                int32_t *mean_table_users) {
  if (!plan) return set_error(DCKV_EINVAL, "plan_memory: null plan");
  if (table_bytes) *table_bytes = plan->dev_bytes;
  if (mean_table_bytes) *mean_table_bytes = (uint64_t)plan->vocab * plan->C * 4;
  if (mean_table_users) {
    std::lock_guard<std::mutex> lk(mt_state().mu);
    auto it = mt_state().tables.find(mt_key(plan));
    *mean_table_users = it == mt_state().tables.end() ? 0 : it->second.users;
  }
  return DCKV_OK;
}

extern "C" int dckv_plan_info(const dckv_plan_t *plan, float *step_out, uint8_t *active_out,
                              uint16_t *freq_out, int32_t *c_active, uint32_t *crc) {
  if (!plan) return set_error(DCKV_EINVAL, "plan_info: null plan");
  if (step_out) std::memcpy(step_out, plan->step.data(), plan->step.size() * 4);
  if (active_out) std::memcpy(active_out, plan->active.data(), plan->active.size());
  if (freq_out) std::memcpy(freq_out, plan->freq.data(), plan->freq.size() * 2);
  if (c_active) *c_active = plan->C_a;
  if (crc) *crc = plan->crc;
  return DCKV_OK;
}

extern "C" int dckv_plan_mean_table(const dckv_plan_t *plan, const float **table, int64_t *rows,
                                    int32_t *col_component) {
  if (!plan) return set_error(DCKV_EINVAL, "plan_mean_table: null plan");
  if (table) *table = plan->mtab;
  if (rows) *rows = plan->vocab;
  if (col_component) {
    int i = 0;
    for (int c = 0; c < plan->C; ++c)
      if (plan->active[c]) col_component[i++] = c;
    for (int c = 0; c < plan->C; ++c)
      if (!plan->active[c]) col_component[i++] = c;
  }
  return DCKV_OK;
}

// ---------------------------------------------------------------------------
// geometry and workspace
// ---------------------------------------------------------------------------
Geometry dckv::geometry(const dckv_plan_t *p, int64_t T) {
  Geometry g{};
  g.T = T;
  g.N = std::max<int64_t>(T - p->keep_head - p->keep_tail, 0);
  g.n_kept = T - g.N;
  g.n_blk = (g.N + kBlock - 1) / kBlock;
  g.G = p->G;
  g.n_groups = g.n_blk * g.G;
  g.N256 = g.n_blk * kBlock;
  g.NM = round_up(g.N, kBM);
  g.n_mtiles = g.NM / kBM;
  g.Ca4 = round_up(std::max(p->C_a, 1), kBN);
  g.esc_cap = std::max<int64_t>(4096, g.N * (int64_t)p->C_a / 16);
  g.rope_hi = std::max<int64_t>(1, (T + 255) / 256);
  g.fixed_bytes = kHeaderBytes + (uint64_t)g.n_kept * p->D * 2 + 4ull * (g.n_groups + 1);
  return g;
}

Layout dckv::layout(const dckv_plan_t *p, const Geometry &g) {
  Layout l{};
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    uint64_t o = off;
    off = align256(off + std::max<uint64_t>(bytes, 1));
    return o;
  };
  l.ctrl = take(sizeof(Ctrl));
  l.sym = take((uint64_t)g.G * g.N256 * kLanes);
  l.halo_a = take((uint64_t)g.n_mtiles * p->C * 4);
  l.halo_b = take((uint64_t)g.n_mtiles * p->C * 4);
  const uint64_t shared_end = off;
  // encode-only region
  uint64_t cap2 = 1;
  while (cap2 < (uint64_t)g.esc_cap) cap2 <<= 1;
  l.esc_raw = take(cap2 * 8);  // room for the bitonic sort's power-of-two padding
  l.esc_sorted = take((uint64_t)g.esc_cap * 8);
  l.scratch = take((uint64_t)g.n_groups * kLanes * (kBlock + 2) * 2);
  l.gwords = take((uint64_t)g.n_groups * 4);
  l.goffs = take((uint64_t)(g.n_groups + 1) * 8);
  const uint64_t enc_end = off;
  // decode-only region (overlaps the encode-only one)
  off = shared_end;
  l.yhat_b = take((uint64_t)g.NM * p->C * 2);
  l.esc_rows = take((uint64_t)g.n_mtiles * 2 * 4);
  l.dhalo = take(2ull * g.n_mtiles * p->C * 4);  // fused dequantisation: left neighbours, first rows
  l.h_b = take((uint64_t)g.NM * p->hidden * 2);
  l.w1_part = take(2ull * g.NM * p->hidden * 4);
  l.rope_lo = take(256ull * kHalf * 8);
  l.rope_hi = take((uint64_t)g.rope_hi * kHalf * 8);
  const uint64_t dec_end = off;
  l.enc_total = enc_end;
  l.total = std::max(enc_end, dec_end);
  return l;
}

extern "C" int dckv_bytes(const dckv_plan_t *plan, int64_t T, uint64_t *max_stream_bytes,
                          uint64_t *workspace_bytes) {
  if (!plan) return set_error(DCKV_EINVAL, "bytes: null plan");
  if (T < 0 || T > (int64_t)0x7FFFFFFF) return set_error(DCKV_EINVAL, "bytes: T out of range");
  if (T > kMaxRows) return set_error(DCKV_EUNSUPPORTED, "bytes: T above 2^18 positions (32-bit operand offsets)");
  Geometry g = geometry(plan, T);
  // a coded position costs at most one 16-bit word or one 8-byte escape record;
  // each substream adds a two-word flush.  An encode refuses more escapes than
  // the workspace holds (esc_cap, DCKV_ECAPACITY), so at most esc_cap records.
  const uint64_t symbols = (uint64_t)g.N * plan->C_a;
  const uint64_t rans_max = 2ull * symbols + 4ull * (uint64_t)g.n_blk * plan->C_a;
  if (rans_max >= 0xFFFFFFFFull || symbols >= 0xFFFFFFFFull)
    return set_error(DCKV_EUNSUPPORTED, "bytes: request too long for 32-bit stream offsets");
  const uint64_t esc_max = std::min<uint64_t>((uint64_t)g.esc_cap, symbols);
  if (max_stream_bytes) *max_stream_bytes = g.fixed_bytes + rans_max + 6ull * esc_max;
  if (workspace_bytes) *workspace_bytes = layout(plan, g).total;
  return DCKV_OK;
}

extern "C" int dckv_workspace_view(const dckv_plan_t *plan, int64_t T, int32_t which, uint64_t *offset,
                                   uint64_t *bytes, int64_t *row_stride) {
  if (!plan || T < 0) return set_error(DCKV_EINVAL, "workspace_view: bad argument");
  Geometry g = geometry(plan, T);
  Layout l = layout(plan, g);
  uint64_t o = 0, b = 0;
  int64_t rs = 0;
  switch (which) {
    case DCKV_VIEW_SYMBOLS: o = l.sym; b = (uint64_t)g.G * g.N256 * kLanes; rs = kLanes; break;
    case DCKV_VIEW_YHAT_B: o = l.yhat_b; b = (uint64_t)g.N * plan->C * 2; rs = plan->C; break;
    case DCKV_VIEW_H_B: o = l.h_b; b = (uint64_t)g.N * plan->hidden * 2; rs = plan->hidden; break;
    default: return set_error(DCKV_EINVAL, "workspace_view: unknown view");
  }
  if (offset) *offset = o;
  if (bytes) *bytes = b;
  if (row_stride) *row_stride = rs;
  return DCKV_OK;
}

// ---------------------------------------------------------------------------
// kernel timing
// ---------------------------------------------------------------------------
namespace {
struct ProfState {
  std::mutex mu;
  bool on = false;
  std::string only;  // time only this kernel (empty: all)
  struct Pending {
    std::string name;
    hipEvent_t a, b;
  };
  std::vector<Pending> pending;
  std::map<std::string, std::pair<double, int64_t>> acc;
};
ProfState &prof() {
  static ProfState s;
  return s;
}
void drain_locked(ProfState &s) {
  for (auto &e : s.pending) {
    float ms = 0.f;
    if (hipEventSynchronize(e.b) == hipSuccess && hipEventElapsedTime(&ms, e.a, e.b) == hipSuccess) {
      auto &slot = s.acc[e.name];
      slot.first += ms;
      slot.second += 1;
    }
    (void)hipEventDestroy(e.a);
    (void)hipEventDestroy(e.b);
  }
  s.pending.clear();
}
}  // namespace

KernelTimer::KernelTimer(const char *name, hipStream_t s) : name_(name), s_(s) {
  ProfState &st = prof();
  if (!st.on) return;
  {
    std::lock_guard<std::mutex> g(st.mu);
    if (!st.only.empty() && st.only != name) return;
  }
  if (hipEventCreate(&a_) != hipSuccess || hipEventCreate(&b_) != hipSuccess) {
    a_ = b_ = nullptr;
    return;
  }
  (void)hipEventRecord(a_, s_);
}

KernelTimer::~KernelTimer() {
  if (!a_) return;
  (void)hipEventRecord(b_, s_);
  ProfState &st = prof();
  std::lock_guard<std::mutex> g(st.mu);
  st.pending.push_back({name_, a_, b_});
  if (st.pending.size() > 4096) drain_locked(st);
}

extern "C" int dckv_profile_enable(int32_t on) {
  prof().on = on != 0;
  return DCKV_OK;
}

extern "C" int dckv_profile_only(const char *kernel) {
  ProfState &s = prof();
  std::lock_guard<std::mutex> g(s.mu);
  s.only = kernel ? kernel : "";
  return DCKV_OK;
}

extern "C" int dckv_profile_reset(void) {
  ProfState &s = prof();
  std::lock_guard<std::mutex> g(s.mu);
  drain_locked(s);
  s.acc.clear();
  return DCKV_OK;
}

extern "C" int dckv_profile_read(const char *kernel, double *total_ms, int64_t *launches) {
  if (!kernel) return set_error(DCKV_EINVAL, "profile_read: null name");
  ProfState &s = prof();
  std::lock_guard<std::mutex> g(s.mu);
  drain_locked(s);
  auto it = s.acc.find(kernel);
  if (total_ms) *total_ms = it == s.acc.end() ? 0.0 : it->second.first;
  if (launches) *launches = it == s.acc.end() ? 0 : it->second.second;
  return DCKV_OK;
}
