// Model loading (copy, LoRA merge, layout), request plans and the layer loop.
//
// One prefill pass per request, no decoding (System1-Omni README,
// introduction).  Sequences are packed without padding; a request with
// branches runs two passes over the same packed buffers: pass A over every
// sequence that is not a branch (prefixes write their full-attention keys and
// values and their final linear-attention state), pass B over the branches,
// which start from that snapshot (RFC #114 section 5).  The readout then runs
// only at the questions' marker rows (sys1rust README, "How it works": the
// head runs only at the positions the answer reads).
#include <algorithm>
#include <initializer_list>
#include <climits>
#include <cstring>
#include <map>
#include <new>
#include <string>
#include <vector>

#include "internal.h"

namespace s1 {

#define S1_TRY(expr, what)                                  \
  do {                                                      \
    hipError_t e_ = (expr);                                 \
    if (e_ != hipSuccess) return set_error(S1_EDEVICE, hip_msg(e_, what)); \
  } while (0)

const char* kernel_class_name(int c) {
  static const char* names[KC_COUNT] = {"embed", "rmsnorm", "gemm_la_in", "la_scan", "gemm_fa_qkv",
                                        "attention", "gemm_o", "gemm_gate_up", "gemm_down", "capture",
                                        "readout", "vocab_lse", "features"};
  return (c >= 0 && c < KC_COUNT) ? names[c] : "?";
}

Profiler::~Profiler() {
  for (hipEvent_t e : ev) (void)hipEventDestroy(e);
}

int Profiler::reserve(int n) {
  while ((int)ev.size() < n) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return S1_EDEVICE;
    ev.push_back(e);
  }
  cls.resize(ev.size());
  return S1_OK;
}

void Profiler::begin(hipStream_t s) {
  used = 0;
  overflow = false;
  mark(-1, s);
}

void Profiler::mark(int c, hipStream_t s) {
  if (used >= (int)ev.size()) {
    overflow = true;
    return;
  }
  (void)hipEventRecord(ev[used], s);
  cls[used++] = c;
}

void Model::drop_decide_graph() {
  if (decide_gexec) (void)hipGraphExecDestroy(decide_gexec);
  if (decide_graph) (void)hipGraphDestroy(decide_graph);
  decide_gexec = nullptr;
  decide_graph = nullptr;
}

Model::~Model() {
  drop_decide_graph();
  delete prof_store;
  for (hipEvent_t e : decide_ev)
    if (e) (void)hipEventDestroy(e);
  if (decide_dev) (void)hipFree(decide_dev);
  for (void* p : allocs) (void)hipFree(p);
  if (own_stream) (void)hipStreamDestroy(own_stream);
}

void* Model::alloc(size_t bytes) {
  void* p = nullptr;
  if (bytes == 0) bytes = 256;
  if (dev_alloc(&p, bytes) != hipSuccess) throw std::bad_alloc();
  allocs.push_back(p);
  return p;
}

void Plan::drop_graph() {
  if (gexec) (void)hipGraphExecDestroy(gexec);
  if (graph) (void)hipGraphDestroy(graph);
  gexec = nullptr;
  graph = nullptr;
}

Plan::~Plan() {
  drop_graph();
  if (dev && dev_owned) (void)hipFree(dev);
  if (cap_dev) (void)hipFree(cap_dev);
  if (inj_dev) (void)hipFree(inj_dev);
  if (feat_dev) (void)hipFree(feat_dev);
}

namespace {

struct TensorTable {
  std::map<std::string, const s1_tensor*> byname;
  const s1_tensor* get(const std::string& n) const {
    auto it = byname.find(n);
    return it == byname.end() ? nullptr : it->second;
  }
};

// Index of dimension i of a rotate-half head after the permutation that puts
// the partner of each column exactly 32 columns later: within every group of
// 64 columns, the first 32 hold dims d and the next 32 hold dims d + hd/2.
int rope_perm(int i, int hd) {
  const int half = hd / 2;
  if (i < half) return 64 * (i / 32) + (i % 32);
  const int j = i - half;
  return 64 * (j / 32) + 32 + (j % 32);
}

class Loader {
 public:
  Loader(Model* m, const TensorTable& tt, hipStream_t s) : m_(m), tt_(tt), s_(s) {}
  ~Loader() {
    for (void* p : scratch_) (void)hipFree(p);
  }

  // Copy (or reference) tensor `name`, checking its shape.
  int fetch(const std::string& name, int64_t rows, int64_t cols, const void** dev) {
    const s1_tensor* t = tt_.get(name);
    if (!t) return set_error(S1_EINVAL, "missing tensor '" + name + "'");
    const int64_t r = t->ndim == 1 ? 1 : t->shape[0];
    const int64_t c = t->ndim == 1 ? t->shape[0] : t->shape[1];
    const int64_t want_r = cols < 0 ? 1 : rows, want_c = cols < 0 ? rows : cols;
    if (t->dtype != m_->cfg.dtype || t->ndim < 1 || t->ndim > 2 || r != want_r || c != want_c ||
        t->data == nullptr)
      return set_error(S1_EINVAL, "tensor '" + name + "' has the wrong dtype, shape or no data");
    const size_t bytes = (size_t)(want_r * want_c) * m_->esz;
    if (t->on_device) {
      *dev = t->data;
      return S1_OK;
    }
    void* p = nullptr;
    if (dev_alloc(&p, bytes) != hipSuccess) {
      (void)hipGetLastError();
      return set_error(S1_ENOMEM, "device allocation for '" + name + "' failed");
    }
    scratch_.push_back(p);
    S1_TRY(hipMemcpy(p, t->data, bytes, hipMemcpyHostToDevice), "copy weights to device");
    *dev = p;
    return S1_OK;
  }

  // Merge the adapter of `name` (if it is a target) into its rows of dst,
  // row o of the [out, in] source going to dst row map[o] (or base + o).
  int projection(const std::string& name, int out_dim, int in_dim, bool target, void* dst,
                 const std::vector<int>& map, const float* gain = nullptr) {
    const void* w = nullptr;
    const void* a = nullptr;
    const void* b = nullptr;
    int rc = fetch(name, out_dim, in_dim, &w);
    if (rc) return rc;
    const int r = m_->cfg.lora_rank;
    if (target) {
      if ((rc = fetch(name + ".lora_A", r, in_dim, &a))) return rc;
      if ((rc = fetch(name + ".lora_B", out_dim, r, &b))) return rc;
    }
    int* dmap = nullptr;
    if (!map.empty()) {
      if (dev_alloc(reinterpret_cast<void**>(&dmap), map.size() * sizeof(int)) != hipSuccess) {
        (void)hipGetLastError();
        return set_error(S1_ENOMEM, "device allocation failed");
      }
      scratch_.push_back(dmap);
      S1_TRY(hipMemcpy(dmap, map.data(), map.size() * sizeof(int), hipMemcpyHostToDevice), "copy row map");
    }
    const float scale = target ? m_->cfg.lora_alpha / (float)r : 0.f;
    S1_TRY(launch_merge(m_->bf16, w, target ? a : nullptr, target ? b : nullptr, dst, out_dim, in_dim,
                        r, scale, dmap, s_, gain),
           "LoRA merge");
    S1_TRY(hipStreamSynchronize(s_), "LoRA merge");
    release();
    return S1_OK;
  }

  // A small [rows, cols] tensor converted to fp32 (convolution taps).
  int taps(const std::string& name, int rows, int cols, float** out) {
    const void* w = nullptr;
    int rc = fetch(name, rows, cols, &w);
    if (rc) return rc;
    *out = static_cast<float*>(m_->alloc((size_t)rows * cols * sizeof(float)));
    S1_TRY(launch_to_f32(m_->bf16, w, *out, (long long)rows * cols, s_), "convolution taps");
    S1_TRY(hipStreamSynchronize(s_), "convolution taps");
    release();
    return S1_OK;
  }

  int norm(const std::string& name, int d, float** out) {
    const void* w = nullptr;
    int rc = fetch(name, d, -1, &w);
    if (rc) return rc;
    *out = static_cast<float*>(m_->alloc((size_t)d * sizeof(float)));
    S1_TRY(launch_to_f32(m_->bf16, w, *out, d, s_), "norm gains");
    S1_TRY(hipStreamSynchronize(s_), "norm gains");
    release();
    return S1_OK;
  }

  void release() {
    for (void* p : scratch_) (void)hipFree(p);
    scratch_.clear();
  }

 private:
  Model* m_;
  const TensorTable& tt_;
  hipStream_t s_;
  std::vector<void*> scratch_;
};

std::vector<int> offset_map(int n, int base) {
  std::vector<int> v(n);
  for (int i = 0; i < n; ++i) v[i] = base + i;
  return v;
}

// Fragment-order copy of a bf16 weight [N, K] for the weight-direct GEMM
// (K a multiple of 64); nothing for fp32 models or other K.
int pack_direct(Model* m, const void* W, int N, int K, void** out, hipStream_t s) {
  if (!m->bf16 || K % 64) return S1_OK;
  *out = m->alloc(frag_bytes(N, K));
  S1_TRY(launch_frag_pack(W, N, K, K, false, *out, s), "pack a weight for the weight-direct GEMM");
  return S1_OK;
}

int load_layers(Model* m, Loader& ld, hipStream_t s) {
  const s1_config& c = m->cfg;
  const int d = c.d_model, F = c.ffn, H = c.la_heads, dk = c.la_dk, dv = c.la_dv;
  const int Hq = c.fa_q_heads, Hkv = c.fa_kv_heads, hd = c.fa_head_dim;
  const uint32_t tg = c.lora_targets;
  int rc;
  for (int l = 0; l < c.n_layers; ++l) {
    LayerW& L = m->layers[l];
    const std::string p = "layers." + std::to_string(l);
    if ((rc = ld.norm(p + ".attn_norm", d, &L.attn_norm))) return rc;
    if ((rc = ld.norm(p + ".ffn_norm", d, &L.ffn_norm))) return rc;
    // with the deferred norm the gains scale the consuming weights' columns
    const float* ga = m->fold ? L.attn_norm : nullptr;
    const float* gf = m->fold ? L.ffn_norm : nullptr;
    if (!L.full) {
      const std::string q = p + ".la";
      const bool gdn = c.la_kind == S1_LA_GDN;
      L.n_in = 2 * H * dk + H * dv + (gdn ? 2 : 1) * H;
      L.w_in = m->alloc((size_t)L.n_in * d * m->esz);
      if ((rc = ld.projection(q + ".q", H * dk, d, tg & S1_LORA_Q, L.w_in, offset_map(H * dk, 0), ga))) return rc;
      if ((rc = ld.projection(q + ".k", H * dk, d, tg & S1_LORA_K, L.w_in, offset_map(H * dk, H * dk), ga)))
        return rc;
      if ((rc = ld.projection(q + ".v", H * dv, d, tg & S1_LORA_V, L.w_in, offset_map(H * dv, 2 * H * dk), ga)))
        return rc;
      if ((rc = ld.projection(q + ".g", H, d, false, L.w_in, offset_map(H, 2 * H * dk + H * dv), ga))) return rc;
      if (gdn) {
        if ((rc = ld.projection(q + ".b", H, d, false, L.w_in, offset_map(H, 2 * H * dk + H * dv + H), ga)))
          return rc;
        if ((rc = ld.taps(q + ".conv", 2 * H * dk + H * dv, 4, &L.conv))) return rc;
      }
      L.k_o = H * dv;
      if ((rc = pack_direct(m, L.w_in, L.n_in, d, &L.w_in_frag, s))) return rc;
      L.w_o = m->alloc((size_t)d * L.k_o * m->esz);
      if ((rc = ld.projection(q + ".o", d, L.k_o, tg & S1_LORA_O, L.w_o, {}))) return rc;
      if ((rc = pack_direct(m, L.w_o, d, L.k_o, &L.w_o_frag, s))) return rc;
    } else {
      const std::string q = p + ".fa";
      L.n_in = (Hq + 2 * Hkv) * hd;
      L.w_in = m->alloc((size_t)L.n_in * d * m->esz);
      std::vector<int> mq(Hq * hd), mk(Hkv * hd);
      for (int h = 0; h < Hq; ++h)
        for (int i = 0; i < hd; ++i) mq[h * hd + i] = h * hd + rope_perm(i, hd);
      for (int h = 0; h < Hkv; ++h)
        for (int i = 0; i < hd; ++i) mk[h * hd + i] = Hq * hd + h * hd + rope_perm(i, hd);
      if ((rc = ld.projection(q + ".q", Hq * hd, d, tg & S1_LORA_Q, L.w_in, mq, ga))) return rc;
      if ((rc = ld.projection(q + ".k", Hkv * hd, d, tg & S1_LORA_K, L.w_in, mk, ga))) return rc;
      if ((rc = ld.projection(q + ".v", Hkv * hd, d, tg & S1_LORA_V, L.w_in,
                              offset_map(Hkv * hd, (Hq + Hkv) * hd), ga))) return rc;
      L.k_o = Hq * hd;
      if ((rc = pack_direct(m, L.w_in, L.n_in, d, &L.w_in_frag, s))) return rc;
      L.w_o = m->alloc((size_t)d * L.k_o * m->esz);
      if ((rc = ld.projection(q + ".o", d, L.k_o, tg & S1_LORA_O, L.w_o, {}))) return rc;
      if ((rc = pack_direct(m, L.w_o, d, L.k_o, &L.w_o_frag, s))) return rc;
    }
    const std::string f = p + ".ffn";
    L.n_gu = 2 * m->ffn_pad;
    L.w_gu = m->alloc((size_t)L.n_gu * d * m->esz);
    S1_TRY(hipMemsetAsync(L.w_gu, 0, (size_t)L.n_gu * d * m->esz, s), "clear gate/up");
    std::vector<int> mg(F), mu(F);
    for (int i = 0; i < F; ++i) {
      mg[i] = 64 * (i / 32) + (i % 32);
      mu[i] = mg[i] + 32;
    }
    if ((rc = ld.projection(f + ".gate", F, d, tg & S1_LORA_GATE, L.w_gu, mg, gf))) return rc;
    if ((rc = ld.projection(f + ".up", F, d, tg & S1_LORA_UP, L.w_gu, mu, gf))) return rc;
    if (m->bf16 && d % 64 == 0 && F % 8 == 0) {   // the weight-direct GEMM's copy
      L.w_gu_frag = m->alloc(frag_bytes(L.n_gu, d));
      S1_TRY(launch_frag_pack(L.w_gu, L.n_gu, d, d, true, L.w_gu_frag, s), "pack gate/up");
    }
    L.w_down = m->alloc((size_t)d * F * m->esz);
    if ((rc = ld.projection(f + ".down", d, F, tg & S1_LORA_DOWN, L.w_down, {}))) return rc;
    if ((rc = pack_direct(m, L.w_down, d, F, &L.w_down_frag, s))) return rc;
  }
  return S1_OK;
}

int alloc_workspace(Model* m) {
  const s1_config& c = m->cfg;
  const long long T = c.max_tokens, d = c.d_model;
  const int H = c.la_heads, Hq = c.fa_q_heads, Hkv = c.fa_kv_heads, hd = c.fa_head_dim;
  m->ld_qkv = std::max(2 * H * c.la_dk + H * c.la_dv, Hq * hd);
  m->ld_att = std::max(H * c.la_dv, Hq * hd);
  m->x = static_cast<float*>(m->alloc(T * d * sizeof(float)));
  m->xn = m->alloc(T * d * m->esz);
  m->qkv = m->alloc(T * m->ld_qkv * m->esz);
  m->lg = static_cast<float*>(m->alloc(T * H * sizeof(float)));
  if (c.la_kind == S1_LA_GDN) {
    const long long Cc = 2LL * H * c.la_dk + (long long)H * c.la_dv;
    m->beta = static_cast<float*>(m->alloc(T * H * sizeof(float)));
    m->qkv2 = m->alloc(T * m->ld_qkv * m->esz);
    m->conv_hist = m->alloc((size_t)std::max(1, m->n_la) * c.max_prefixes * 3 * Cc * m->esz);
  }
  m->att = m->alloc(T * m->ld_att * m->esz);
  m->hbuf = m->alloc(T * (long long)c.ffn * m->esz);
  m->kc = m->alloc((size_t)std::max(1, m->n_fa) * T * Hkv * hd * m->esz);
  m->vc = m->alloc((size_t)std::max(1, m->n_fa) * T * Hkv * hd * m->esz);
  m->states = static_cast<float*>(m->alloc((size_t)std::max(1, m->n_la) * c.max_prefixes * H *
                                           c.la_dk * c.la_dv * sizeof(float)));
  if (m->bf16) {
    // chunk-parallel scan workspace, shared by all linear layers (one layer at a time)
    m->max_chunks = (int)((T + 63) / 64) + c.max_seqs;
    m->cstates = static_cast<float*>(m->alloc((size_t)m->max_chunks * H * c.la_dk * c.la_dv * sizeof(float)));
    m->gamma = static_cast<float*>(m->alloc((size_t)m->max_chunks * H * sizeof(float)));
    if (c.la_kind == S1_LA_GDN) m->gdn_ws = static_cast<float*>(m->alloc(gdn_ws_bytes(m->max_chunks, H)));
  }
  if (m->fold) {
    m->ss_ld = (int)((T + 31) / 32 * 32);
    m->rstd = static_cast<float*>(m->alloc(T * sizeof(float)));
    m->ssq = static_cast<float*>(m->alloc((size_t)((d + 31) / 32) * m->ss_ld * sizeof(float)));
    const size_t nt = (size_t)(T + 31) / 32 + 1;   // row blocks of the smallest tile
    m->tickets = static_cast<unsigned int*>(m->alloc(nt * sizeof(unsigned int)));
    if (hipMemset(m->tickets, 0, nt * sizeof(unsigned int)) != hipSuccess)
      return set_error(S1_EDEVICE, "clear the row-block tickets");
  }
  m->split_max_rows = (int)std::min<long long>(T, 2048);
  m->splitws_elems = 4LL * m->split_max_rows * d;
  m->splitws = static_cast<float*>(m->alloc(m->splitws_elems * sizeof(float)));
  m->rope = static_cast<float2*>(m->alloc((size_t)c.max_positions * (hd / 2) * sizeof(float2)));
  return S1_OK;
}

}  // namespace

int load_model(const s1_config* cfg, const s1_tensor* tensors, int n, hipStream_t user_stream,
               Model** out) {
  int rc = validate_config(cfg);
  if (rc) return rc;
  if (n < 0 || (n > 0 && tensors == nullptr)) return set_error(S1_EINVAL, "tensor table is NULL");
  TensorTable tt;
  for (int i = 0; i < n; ++i) {
    if (tensors[i].name == nullptr) return set_error(S1_EINVAL, "tensor with a NULL name");
    tt.byname[tensors[i].name] = &tensors[i];
  }
  Model* m = new (std::nothrow) Model();
  if (!m) return set_error(S1_ENOMEM, "host allocation failed");
  m->cfg = *cfg;
  m->bf16 = cfg->dtype == S1_BF16;
  m->esz = m->bf16 ? 2 : 4;
  m->ffn_pad = (cfg->ffn + 31) / 32 * 32;
  // the deferred RMSNorm: bf16 rows that the fused norm kernels hold (d % 4,
  // d <= 16,384) with at most 256 partial sums of 32 columns
  m->fold = m->bf16 && cfg->d_model % 32 == 0 && cfg->d_model <= 256 * 32;
  if (hipGetDevice(&m->device) != hipSuccess) {
    delete m;
    return set_error(S1_EDEVICE, "no HIP device");
  }
  int n_cu = 0;
  if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, m->device) == hipSuccess && n_cu > 0)
    m->n_cu = n_cu;
  if (hipStreamCreateWithFlags(&m->own_stream, hipStreamNonBlocking) != hipSuccess) {
    delete m;
    return set_error(S1_EDEVICE, "stream creation failed");
  }
  hipStream_t s = user_stream ? user_stream : m->own_stream;
  m->layers.resize(cfg->n_layers);
  for (int l = 0; l < cfg->n_layers; ++l) {
    LayerW& L = m->layers[l];
    L.full = (l % cfg->full_every) == cfg->full_every - 1;
    if (L.full) L.fa_idx = m->n_fa++;
    else L.la_idx = m->n_la++;
  }
  try {
    Loader ld(m, tt, s);
    const void* e = nullptr;
    rc = ld.fetch("embed", cfg->vocab, cfg->d_model, &e);
    if (!rc) {
      const size_t bytes = (size_t)cfg->vocab * cfg->d_model * m->esz;
      m->embed = m->alloc(bytes);
      if (hipMemcpyAsync(m->embed, e, bytes, hipMemcpyDeviceToDevice, s) != hipSuccess ||
          hipStreamSynchronize(s) != hipSuccess)
        rc = set_error(S1_EDEVICE, "copy embedding");
      ld.release();
    }
    if (!rc) rc = ld.norm("final_norm", cfg->d_model, &m->final_norm);
    if (!rc) rc = load_layers(m, ld, s);
    if (!rc) rc = alloc_workspace(m);
    if (!rc) {
      if (launch_rope_table(m->rope, (int)cfg->max_positions, cfg->fa_head_dim, cfg->rope_base, s) !=
              hipSuccess ||
          hipStreamSynchronize(s) != hipSuccess)
        rc = set_error(S1_EDEVICE, "rope table");
    }
  } catch (const std::bad_alloc&) {
    rc = set_error(S1_ENOMEM, "device allocation failed while loading the model");
  }
  if (rc) {
    (void)hipStreamSynchronize(s);
    delete m;
    return rc;
  }
  *out = m;
  return S1_OK;
}

// ------------------------------------------------------------------ plans
int create_plan(Model* m, const s1_batch* b, Plan** out, int opts_capacity, bool model_block, size_t extra_bytes) {
  int rc = validate_batch(&m->cfg, b);
  if (rc) return rc;
  Plan* p = new (std::nothrow) Plan();
  if (!p) return set_error(S1_ENOMEM, "host allocation failed");
  p->m = m;
  const int n = b->n_seqs;
  p->n_seqs = n;
  p->T = n > 0 ? b->cu_seqlens[n] : 0;
  p->Q = b->n_questions;
  p->total_opts = p->Q > 0 ? b->opt_offsets[p->Q] : 0;
  for (int j = 0; j < p->Q; ++j) p->max_k = std::max(p->max_k, b->opt_offsets[j + 1] - b->opt_offsets[j]);

  auto pre = [&](int i) { return b->prefix_of ? b->prefix_of[i] : -1; };
  std::vector<int> slot(n, -1);
  int n_slots = 0;
  for (int i = 0; i < n; ++i)
    if (pre(i) >= 0 && slot[pre(i)] < 0) slot[pre(i)] = n_slots++;
  // internal order: pass A (non-branches) then pass B (branches, those of
  // one prefix next to each other so that they can share its key sweep)
  std::vector<int> order[2];
  for (int i = 0; i < n; ++i) order[pre(i) >= 0 ? 1 : 0].push_back(i);
  std::stable_sort(order[1].begin(), order[1].end(), [&](int a, int c) { return slot[pre(a)] < slot[pre(c)]; });
  std::vector<int> row0(n, 0);
  p->row_of.assign(p->T, 0);
  p->pass_of_row.assign(p->T, 0);
  std::vector<int32_t> ids(p->T), pos(p->T);
  int r = 0;
  p->n_passes = order[1].empty() ? 1 : 2;
  for (int ps = 0; ps < 2; ++ps) {
    p->pass[ps].r0 = r;
    for (int i : order[ps]) {
      row0[i] = r;
      const int len = b->cu_seqlens[i + 1] - b->cu_seqlens[i];
      const int P = pre(i) >= 0 ? b->cu_seqlens[pre(i) + 1] - b->cu_seqlens[pre(i)] : 0;
      for (int t = 0; t < len; ++t) {
        p->row_of[b->cu_seqlens[i] + t] = r + t;
        p->pass_of_row[r + t] = ps;
        ids[r + t] = b->token_ids[b->cu_seqlens[i] + t];
        pos[r + t] = P + t;
      }
      r += len;
    }
    p->pass[ps].T = r - p->pass[ps].r0;
    p->pass[ps].n_seqs = (int)order[ps].size();
  }
  std::vector<ScanSeq> scan[2];
  // attention: the split plan (keys cut into pieces, branch prefixes shared)
  // for the default schedule, the unsplit one for the row-invariant mode
  AttnPlanHost aplan[2], aplan_inv[2];
  for (int ps = 0; ps < 2; ++ps) {
    std::vector<int> lens;
    std::vector<AttnSeq> attn;
    for (const int i : order[ps]) lens.push_back(b->cu_seqlens[i + 1] - b->cu_seqlens[i]);
    const int bq = attn_block_rows(m->bf16, lens.data(), (int)lens.size(), m->cfg.fa_q_heads);
    p->pass[ps].attn_rows = bq;
    for (size_t k = 0; k < order[ps].size(); ++k) {
      const int i = order[ps][k];
      const int len = lens[k];
      const int pi = pre(i);
      const int P = pi >= 0 ? b->cu_seqlens[pi + 1] - b->cu_seqlens[pi] : 0;
      scan[ps].push_back({row0[i], len, pi >= 0 ? slot[pi] : -1, slot[i]});
      p->pass[ps].max_len = std::max(p->pass[ps].max_len, len);
      attn.push_back({row0[i], len, row0[i], pi >= 0 ? row0[pi] : 0, P});
    }
    const int r0 = p->pass[ps].r0, Tp = p->pass[ps].T, Hq = m->cfg.fa_q_heads;
    plan_attention(attn.data(), (int)attn.size(), r0, Tp, Hq, bq, m->bf16 ? -1 : 0, m->n_cu, &aplan[ps]);
    plan_attention(attn.data(), (int)attn.size(), r0, Tp, Hq, bq, 0, m->n_cu, &aplan_inv[ps]);
  }
  // chunk-parallel scan when a pass has few (sequence, head) chains; the
  // chunk lists are built for every bf16 pass, since the row-invariant mode
  // runs every pass chunk-parallel
  std::vector<ScanSeq> chunks[2];
  std::vector<ChunkSeq> cseqs[2];
  for (int ps = 0; ps < 2; ++ps) {
    const long long chains = (long long)order[ps].size() * m->cfg.la_heads;
    p->pass[ps].chunked = m->bf16 && !order[ps].empty() && chains < 192;
    if (!m->bf16 || order[ps].empty()) continue;
    for (size_t k = 0; k < order[ps].size(); ++k) {
      const ScanSeq& sq = scan[ps][k];
      ChunkSeq cs{(int)chunks[ps].size(), 0, sq.s_in, sq.s_out};
      for (int t0 = 0; t0 < sq.len; t0 += 64) {
        const int id = (int)chunks[ps].size();
        chunks[ps].push_back({sq.row0 + t0, std::min(64, sq.len - t0), id, id});
        ++cs.nc;
      }
      // an empty sequence that keeps a state needs the separate state scan
      p->pass[ps].max_nc = std::max(p->pass[ps].max_nc, cs.nc == 0 && cs.s_out >= 0 ? INT_MAX : cs.nc);
      cseqs[ps].push_back(cs);
    }
  }
  if (m->cfg.la_kind == S1_LA_GDN)
    for (int i = 0; i < n; ++i)
      if (slot[i] >= 0 && b->cu_seqlens[i + 1] == b->cu_seqlens[i]) {
        delete p;
        return set_error(S1_EINVAL, "a prefix of a Gated DeltaNet model needs at least one token");
      }
  // Gated DeltaNet: every sequence with its first chunk, and each row's
  // sequence (pass-local), for the convolution and the scan
  std::vector<GdnSeq> gseqs[2];
  std::vector<int32_t> rowseq[2];
  for (int ps = 0; ps < 2 && m->cfg.la_kind == S1_LA_GDN; ++ps) {
    rowseq[ps].assign(p->pass[ps].T, 0);
    for (size_t k = 0; k < order[ps].size(); ++k) {
      const ScanSeq& sq = scan[ps][k];
      gseqs[ps].push_back({sq.row0, sq.len, cseqs[ps][k].c0, sq.s_in, sq.s_out});
      for (int t = 0; t < sq.len; ++t) rowseq[ps][sq.row0 - p->pass[ps].r0 + t] = (int32_t)k;
    }
  }
  std::vector<int32_t> qrow(p->Q);
  for (int j = 0; j < p->Q; ++j) qrow[j] = row0[b->q_seq[j]] + b->q_marker[j];

  // one device block for every array of the plan
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  const size_t o_ids = take(p->T * 4), o_pos = take(p->T * 4), o_qrow = take(p->Q * 4);
  const size_t o_off = take((p->Q + 1) * 4), o_opt = take(std::max(p->total_opts, opts_capacity) * 4);
  const size_t o_qt = take(p->Q);
  size_t o_scan[2], o_attn[2], o_blk[2], o_chk[2], o_cseq[2], o_gseq[2], o_rseq[2];
  size_t o_blki[2], o_rslot[2], o_rnp[2], o_comb[2], o_pO[2], o_pML[2];
  const int Hq = m->cfg.fa_q_heads, hd = m->cfg.fa_head_dim;
  for (int ps = 0; ps < 2; ++ps) {
    const AttnPlanHost& ap = aplan[ps];
    o_scan[ps] = take(scan[ps].size() * sizeof(ScanSeq));
    o_attn[ps] = take(ap.seqs.size() * sizeof(AttnSeq));
    o_blk[ps] = take(ap.blocks.size() * sizeof(AttnBlock));
    o_blki[ps] = take(aplan_inv[ps].blocks.size() * sizeof(AttnBlock));
    o_rslot[ps] = take(ap.row_slot.size() * 4);
    o_rnp[ps] = take(ap.row_np.size() * 4);
    o_comb[ps] = take(ap.comb_rows.size() * 4);
    o_chk[ps] = take(chunks[ps].size() * sizeof(ScanSeq));
    o_cseq[ps] = take(cseqs[ps].size() * sizeof(ChunkSeq));
    o_gseq[ps] = take(gseqs[ps].size() * sizeof(GdnSeq));
    o_rseq[ps] = take(rowseq[ps].size() * sizeof(int32_t));
  }
  const size_t host_bytes = off;   // partial results need no upload
  for (int ps = 0; ps < 2; ++ps) {
    o_pO[ps] = take((size_t)aplan[ps].slots * Hq * hd * 4);
    o_pML[ps] = take((size_t)aplan[ps].slots * Hq * 8);
  }
  const size_t o_extra = take(extra_bytes);
  std::vector<char> host(host_bytes, 0);
  auto put = [&](size_t o, const void* src, size_t bytes) {
    if (bytes) std::memcpy(host.data() + o, src, bytes);
  };
  put(o_ids, ids.data(), p->T * 4);
  put(o_pos, pos.data(), p->T * 4);
  put(o_qrow, qrow.data(), p->Q * 4);
  if (p->Q > 0) {
    put(o_off, b->opt_offsets, (p->Q + 1) * 4);
    put(o_opt, b->opt_ids, p->total_opts * 4);
    put(o_qt, b->q_type, p->Q);
  }
  for (int ps = 0; ps < 2; ++ps) {
    put(o_scan[ps], scan[ps].data(), scan[ps].size() * sizeof(ScanSeq));
    const AttnPlanHost& ap = aplan[ps];
    put(o_attn[ps], ap.seqs.data(), ap.seqs.size() * sizeof(AttnSeq));
    put(o_blk[ps], ap.blocks.data(), ap.blocks.size() * sizeof(AttnBlock));
    put(o_blki[ps], aplan_inv[ps].blocks.data(), aplan_inv[ps].blocks.size() * sizeof(AttnBlock));
    put(o_rslot[ps], ap.row_slot.data(), ap.row_slot.size() * 4);
    put(o_rnp[ps], ap.row_np.data(), ap.row_np.size() * 4);
    put(o_comb[ps], ap.comb_rows.data(), ap.comb_rows.size() * 4);
    put(o_chk[ps], chunks[ps].data(), chunks[ps].size() * sizeof(ScanSeq));
    put(o_cseq[ps], cseqs[ps].data(), cseqs[ps].size() * sizeof(ChunkSeq));
    put(o_gseq[ps], gseqs[ps].data(), gseqs[ps].size() * sizeof(GdnSeq));
    put(o_rseq[ps], rowseq[ps].data(), rowseq[ps].size() * sizeof(int32_t));
  }
  if (model_block) {
    // the model's block, grown only when this request needs more; the
    // previous call synchronised its stream, so nothing still reads it
    if (m->decide_bytes < off) {
      if (m->decide_dev) (void)hipFree(m->decide_dev);
      m->decide_dev = nullptr;
      m->decide_bytes = 0;
      const size_t want = std::max<size_t>(off, 1 << 20);
      if (dev_alloc(&m->decide_dev, want) != hipSuccess) {
        (void)hipGetLastError();
        m->decide_dev = nullptr;
        delete p;
        return set_error(S1_ENOMEM, "device allocation for the request failed");
      }
      m->decide_bytes = want;
    }
    p->dev = m->decide_dev;
    p->dev_owned = false;
  } else if (dev_alloc(&p->dev, std::max<size_t>(off, 256)) != hipSuccess) {
    (void)hipGetLastError();
    p->dev = nullptr;
    delete p;
    return set_error(S1_ENOMEM, "device allocation for the plan failed");
  }
  if (hipMemcpy(p->dev, host.data(), host_bytes, hipMemcpyHostToDevice) != hipSuccess) {
    delete p;
    return set_error(S1_EDEVICE, "copy plan to device");
  }
  char* dv = static_cast<char*>(p->dev);
  p->extra = dv + o_extra;
  p->ids = reinterpret_cast<int32_t*>(dv + o_ids);
  p->pos = reinterpret_cast<int32_t*>(dv + o_pos);
  p->q_row = reinterpret_cast<int32_t*>(dv + o_qrow);
  p->opt_off = reinterpret_cast<int32_t*>(dv + o_off);
  p->opt_ids = reinterpret_cast<int32_t*>(dv + o_opt);
  p->q_type = reinterpret_cast<uint8_t*>(dv + o_qt);
  for (int ps = 0; ps < 2; ++ps) {
    p->pass[ps].scan = reinterpret_cast<ScanSeq*>(dv + o_scan[ps]);
    p->pass[ps].attn = reinterpret_cast<AttnSeq*>(dv + o_attn[ps]);
    p->pass[ps].blocks = reinterpret_cast<AttnBlock*>(dv + o_blk[ps]);
    p->pass[ps].n_blocks = (int)aplan[ps].blocks.size();
    p->pass[ps].blocks_inv = reinterpret_cast<AttnBlock*>(dv + o_blki[ps]);
    p->pass[ps].n_blocks_inv = (int)aplan_inv[ps].blocks.size();
    p->pass[ps].comb_rows = reinterpret_cast<int32_t*>(dv + o_comb[ps]);
    p->pass[ps].n_comb = (int)aplan[ps].comb_rows.size();
    p->pass[ps].attn_part.row_slot = reinterpret_cast<int32_t*>(dv + o_rslot[ps]);
    p->pass[ps].attn_part.row_np = reinterpret_cast<int32_t*>(dv + o_rnp[ps]);
    p->pass[ps].attn_part.row_base = p->pass[ps].r0;
    p->pass[ps].attn_part.pO = reinterpret_cast<float*>(dv + o_pO[ps]);
    p->pass[ps].attn_part.pML = reinterpret_cast<float2*>(dv + o_pML[ps]);
    p->pass[ps].chunks = reinterpret_cast<ScanSeq*>(dv + o_chk[ps]);
    p->pass[ps].n_chunks = (int)chunks[ps].size();
    p->pass[ps].cseqs = reinterpret_cast<ChunkSeq*>(dv + o_cseq[ps]);
    p->pass[ps].gseqs = reinterpret_cast<GdnSeq*>(dv + o_gseq[ps]);
    p->pass[ps].row_seq = reinterpret_cast<int32_t*>(dv + o_rseq[ps]);
  }
  if (p->pass[0].n_chunks + p->pass[1].n_chunks > 0 &&
      std::max(p->pass[0].n_chunks, p->pass[1].n_chunks) > m->max_chunks) {
    delete p;
    return set_error(S1_EBUDGET, "request needs more scan chunks than the workspace holds");
  }
  *out = p;
  return S1_OK;
}

// ------------------------------------------------------ length buckets
int create_bucket_plan(Model* m, int T_b, int Q_b, int O_b, Plan** out) {
  const s1_config& c = m->cfg;
  if (T_b < 1 || Q_b < 1 || O_b < 2 || O_b < 2 * Q_b)
    return set_error(S1_EINVAL, "bucket: need tokens >= 1, questions >= 1 and options >= 2 per question");
  if (c.vocab < 2) return set_error(S1_EINVAL, "bucket: placeholder questions need a vocabulary of >= 2 ids");
  if (T_b > c.max_tokens || T_b > c.max_positions || Q_b > c.max_questions || O_b > (1 << 28) - 2 * Q_b)
    return set_error(S1_EBUDGET, "bucket exceeds the model's budgets");
  // a placeholder request of the bucket's shape: token 0 everywhere, every
  // question a two-way choice at row 0
  std::vector<int32_t> cu = {0, T_b}, ids(T_b, 0), qs(Q_b, 0), qm(Q_b, 0), off(Q_b + 1), opt(2 * Q_b);
  std::vector<uint8_t> qt(Q_b, S1_CHOICE);
  for (int j = 0; j <= Q_b; ++j) off[j] = 2 * j;
  for (int j = 0; j < Q_b; ++j) {
    opt[2 * j] = 0;
    opt[2 * j + 1] = 1;
  }
  s1_batch b{1, cu.data(), ids.data(), nullptr, Q_b, qs.data(), qm.data(), qt.data(), off.data(), opt.data()};
  // the option slot holds a request's O_b options plus two placeholder
  // options for every question slot it leaves unused
  const int cap = O_b + 2 * Q_b;
  Plan* p = nullptr;
  const int rc = create_plan(m, &b, &p, cap);
  if (rc) return rc;
  p->bucket = true;
  p->bucket_opts = O_b;
  p->opts_cap = cap;
  p->max_k = c.max_options;     // the readout's LDS is sized once, at capture
  *out = p;
  return S1_OK;
}

int update_bucket_plan(Plan* p, const s1_batch* b) {
  if (!p->bucket) return set_error(S1_EINVAL, "plan was not created for a length bucket");
  const Model* m = p->m;
  int rc = validate_batch(&m->cfg, b);
  if (rc) return rc;
  if (b->n_seqs != 1 || (b->prefix_of && b->prefix_of[0] >= 0))
    return set_error(S1_EINVAL, "a bucket takes one sequence without a prefix");
  const int L = b->cu_seqlens[1] - b->cu_seqlens[0];
  const int Q = b->n_questions;
  const int nopt = Q > 0 ? b->opt_offsets[Q] : 0;
  if (L > p->T || Q > p->Q || nopt > p->bucket_opts)
    return set_error(S1_EBUDGET, "request exceeds the bucket (tokens, questions or options)");
  // the request, then padding: token 0 after its end (rows past L never
  // reach a real row: every mixer is causal), two-way placeholder questions
  // at row 0 after its questions
  std::vector<int32_t> ids(p->T, 0), qrow(p->Q, 0), off(p->Q + 1), opt;
  std::vector<uint8_t> qt(p->Q, S1_CHOICE);
  for (int t = 0; t < L; ++t) ids[t] = b->token_ids[b->cu_seqlens[0] + t];
  opt.reserve(nopt + 2 * (p->Q - Q));
  off[0] = 0;
  for (int j = 0; j < p->Q; ++j) {
    if (j < Q) {
      qrow[j] = b->q_marker[j];
      qt[j] = b->q_type[j];
      for (int k = b->opt_offsets[j]; k < b->opt_offsets[j + 1]; ++k) opt.push_back(b->opt_ids[k]);
    } else {
      opt.push_back(0);
      opt.push_back(1);
    }
    off[j + 1] = (int32_t)opt.size();
  }
  if ((int)opt.size() > p->opts_cap) return set_error(S1_EBUDGET, "bucket: options exceed the plan's option slot");
  hipError_t e = hipMemcpy(p->ids, ids.data(), 4 * ids.size(), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(p->q_row, qrow.data(), 4 * qrow.size(), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(p->opt_off, off.data(), 4 * off.size(), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(p->opt_ids, opt.data(), 4 * opt.size(), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(p->q_type, qt.data(), qt.size(), hipMemcpyHostToDevice);
  if (e != hipSuccess) return set_error(S1_EDEVICE, hip_msg(e, "bucket update"));
  p->total_opts = (int)opt.size();
  p->real_T = L;
  p->real_Q = Q;
  return S1_OK;
}

int set_capture(Plan* p, int n_rows, const int32_t* rows, float* d_hidden) {
  p->drop_graph();
  if (p->cap_dev) {
    (void)hipFree(p->cap_dev);
    p->cap_dev = nullptr;
  }
  p->n_cap = 0;
  p->cap_out = nullptr;
  for (auto& ps : p->pass) ps.n_cap = 0;
  if (n_rows <= 0) return S1_OK;
  if (rows == nullptr || d_hidden == nullptr) return set_error(S1_EINVAL, "capture rows or buffer is NULL");
  std::vector<int32_t> lists[2][2];   // [pass][rows | dst]
  for (int j = 0; j < n_rows; ++j) {
    if (rows[j] < 0 || rows[j] >= p->T) return set_error(S1_EINVAL, "capture row out of range");
    const int r = p->row_of[rows[j]];
    const int ps = p->pass_of_row[r];
    lists[ps][0].push_back(r);
    lists[ps][1].push_back(j);
  }
  if (dev_alloc(&p->cap_dev, 8 * (size_t)n_rows + 512) != hipSuccess) {
    (void)hipGetLastError();
    return set_error(S1_ENOMEM, "device allocation for capture failed");
  }
  int32_t* d = static_cast<int32_t*>(p->cap_dev);
  for (int ps = 0; ps < 2; ++ps) {
    const int k = (int)lists[ps][0].size();
    if (k) {
      if (hipMemcpy(d, lists[ps][0].data(), 4 * k, hipMemcpyHostToDevice) != hipSuccess ||
          hipMemcpy(d + k, lists[ps][1].data(), 4 * k, hipMemcpyHostToDevice) != hipSuccess)
        return set_error(S1_EDEVICE, "copy capture rows");
    }
    p->pass[ps].cap_rows = d;
    p->pass[ps].cap_dst = d + k;
    p->pass[ps].n_cap = k;
    d += 2 * k;
  }
  p->n_cap = n_rows;
  p->cap_out = d_hidden;
  return S1_OK;
}

int set_layer_inputs(Plan* p, int n_rows, const int32_t* rows, const float* d_src) {
  p->drop_graph();
  if (p->inj_dev) {
    (void)hipFree(p->inj_dev);
    p->inj_dev = nullptr;
  }
  p->n_inj = 0;
  p->inj_src = nullptr;
  for (auto& ps : p->pass) ps.n_inj = 0;
  if (n_rows <= 0) return S1_OK;
  if (rows == nullptr || d_src == nullptr) return set_error(S1_EINVAL, "layer-input rows or buffer is NULL");
  std::vector<int32_t> lists[2][2];   // [pass][rows | index]
  std::vector<char> seen(p->T, 0);
  for (int j = 0; j < n_rows; ++j) {
    if (rows[j] < 0 || rows[j] >= p->T) return set_error(S1_EINVAL, "layer-input row out of range");
    if (seen[rows[j]]) return set_error(S1_EINVAL, "layer-input row listed twice");
    seen[rows[j]] = 1;
    const int r = p->row_of[rows[j]];
    const int ps = p->pass_of_row[r];
    lists[ps][0].push_back(r);
    lists[ps][1].push_back(j);
  }
  if (dev_alloc(&p->inj_dev, 8 * (size_t)n_rows + 512) != hipSuccess) {
    (void)hipGetLastError();
    p->inj_dev = nullptr;
    return set_error(S1_ENOMEM, "device allocation for layer inputs failed");
  }
  int32_t* d = static_cast<int32_t*>(p->inj_dev);
  for (int ps = 0; ps < 2; ++ps) {
    const int k = (int)lists[ps][0].size();
    if (k) {
      if (hipMemcpy(d, lists[ps][0].data(), 4 * k, hipMemcpyHostToDevice) != hipSuccess ||
          hipMemcpy(d + k, lists[ps][1].data(), 4 * k, hipMemcpyHostToDevice) != hipSuccess)
        return set_error(S1_EDEVICE, "copy layer-input rows");
    }
    p->pass[ps].inj_rows = d;
    p->pass[ps].inj_idx = d + k;
    p->pass[ps].n_inj = k;
    d += 2 * k;
  }
  p->n_inj = n_rows;
  p->inj_src = d_src;
  return S1_OK;
}

// --------------------------------------------------------------- features
namespace {
size_t al256(size_t b) { return (b + 255) / 256 * 256; }
}  // namespace

size_t FeatHost::meta_bytes() const {
  return al256(4 * rows.size()) + al256(4 * t_ri.size()) + al256(4 * t_tok.size()) + al256(4 * cand_off.size()) +
         al256(4 * grp_off.size()) + al256(4 * grp_cands.size());
}

hipError_t FeatHost::upload(void* dst, FeatArgs* a, hipStream_t s) const {
  char* d = static_cast<char*>(dst);
  const std::vector<int32_t>* v[6] = {&rows, &t_ri, &t_tok, &cand_off, &grp_off, &grp_cands};
  const int32_t* ptr[6];
  for (int i = 0; i < 6; ++i) {
    ptr[i] = reinterpret_cast<const int32_t*>(d);
    if (!v[i]->empty()) {
      const hipError_t e = hipMemcpyAsync(d, v[i]->data(), 4 * v[i]->size(), hipMemcpyHostToDevice, s);
      if (e != hipSuccess) return e;
    }
    d += al256(4 * v[i]->size());
  }
  a->R = (int)rows.size();
  a->n_targets = (int)t_tok.size();
  a->n_groups = grp_off.empty() ? 0 : (int)grp_off.size() - 1;
  a->rows = ptr[0];
  a->t_ri = ptr[1];
  a->t_tok = ptr[2];
  a->cand_off = ptr[3];
  a->grp_off = ptr[4];
  a->grp_cands = ptr[5];
  return hipSuccess;
}

int build_features(int n_rows, const std::vector<int>* row_map, int V, int n_targets, const int32_t* rows,
                   const int32_t* tokens, int n_cands, const int32_t* cand_offsets, const int32_t* cand_group,
                   const char* who, FeatHost* out) {
  const std::string w(who);
  if (n_targets < 0 || n_cands < 0) return set_error(S1_EINVAL, w + ": negative count");
  if (n_targets > 0 && (!rows || !tokens)) return set_error(S1_EINVAL, w + ": target arrays are NULL");
  if (n_cands > 0 && (!cand_offsets || !cand_group)) return set_error(S1_EINVAL, w + ": candidate arrays are NULL");
  FeatHost h;
  std::vector<int32_t> mapped(n_targets);
  for (int t = 0; t < n_targets; ++t) {
    if (rows[t] < 0 || rows[t] >= n_rows) return set_error(S1_EINVAL, w + ": target row out of range");
    if (tokens[t] < 0 || tokens[t] >= V) return set_error(S1_EINVAL, w + ": target token out of range");
    mapped[t] = row_map ? (*row_map)[rows[t]] : rows[t];
  }
  h.rows = mapped;
  std::sort(h.rows.begin(), h.rows.end());
  h.rows.erase(std::unique(h.rows.begin(), h.rows.end()), h.rows.end());
  h.t_ri.resize(n_targets);
  for (int t = 0; t < n_targets; ++t)
    h.t_ri[t] = (int32_t)(std::lower_bound(h.rows.begin(), h.rows.end(), mapped[t]) - h.rows.begin());
  h.t_tok.assign(tokens, tokens + n_targets);
  if (n_cands > 0) {
    if (cand_offsets[0] < 0) return set_error(S1_EINVAL, w + ": candidate offsets must start at >= 0");
    for (int c = 0; c < n_cands; ++c)
      if (cand_offsets[c + 1] < cand_offsets[c]) return set_error(S1_EINVAL, w + ": candidate offsets decrease");
    if (cand_offsets[n_cands] > n_targets) return set_error(S1_EINVAL, w + ": candidate offsets exceed the targets");
    h.cand_off.assign(cand_offsets, cand_offsets + n_cands + 1);
    std::vector<int32_t> order(n_cands);
    for (int c = 0; c < n_cands; ++c) order[c] = c;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return cand_group[a] < cand_group[b]; });
    h.grp_cands = order;
    h.grp_off.push_back(0);
    for (int i = 1; i <= n_cands; ++i)
      if (i == n_cands || cand_group[order[i]] != cand_group[order[i - 1]]) h.grp_off.push_back(i);
  }
  h.n_cands = n_cands;
  *out = std::move(h);
  return S1_OK;
}

int set_features(Plan* p, const s1_features* f, float* d_logp, float* d_cand_lp, float* d_cand_norm) {
  p->drop_graph();
  if (p->feat_dev) {
    (void)hipFree(p->feat_dev);
    p->feat_dev = nullptr;
  }
  p->feat = FeatArgs();
  p->feat_ws = nullptr;
  p->feat_logp = p->feat_cand_lp = p->feat_cand_norm = nullptr;
  if (!f || f->n_targets == 0) return S1_OK;
  const Model* m = p->m;
  const s1_config& c = m->cfg;
  if (!feat_shape_ok(m->bf16, c.d_model))
    return set_error(S1_EINVAL, "features: d_model must be a multiple of 128 (bf16) or 4 (fp32)");
  if (!d_logp || (f->n_cands > 0 && (!d_cand_lp || !d_cand_norm)))
    return set_error(S1_EINVAL, "features: output buffers are NULL");
  FeatHost h;
  int rc = build_features(p->T, &p->row_of, c.vocab, f->n_targets, f->rows, f->tokens, f->n_cands,
                          f->cand_offsets, f->cand_group, "features", &h);
  if (rc) return rc;
  const FeatWs w = feat_ws_layout(m->bf16, (int)h.rows.size(), c.vocab, c.d_model);
  const size_t meta = h.meta_bytes();
  if (dev_alloc(&p->feat_dev, meta + w.bytes + 256) != hipSuccess) {
    (void)hipGetLastError();
    p->feat_dev = nullptr;
    return set_error(S1_ENOMEM, "device allocation for features failed");
  }
  FeatArgs a;
  hipError_t e = h.upload(p->feat_dev, &a, nullptr);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return set_error(S1_EDEVICE, hip_msg(e, "copy feature metadata"));
  p->feat = a;
  p->feat_ws = static_cast<char*>(p->feat_dev) + meta;
  p->feat_logp = d_logp;
  p->feat_cand_lp = d_cand_lp;
  p->feat_cand_norm = d_cand_norm;
  return S1_OK;
}

// ---------------------------------------------------------------- forward
#define MARK(cls)                            \
  do {                                       \
    if (m->prof) m->prof->mark((cls), s);    \
  } while (0)

namespace {

// The FFN gate/up projection runs on the weight-direct GEMM.  Its launches
// are bound by the operand stream into each CU (BM + BN operand rows per K
// step: 512 for 128 x 384 and 256 x 256, 448 for 192 x 256), so the time
// follows the number of waves of workgroups times that panel; the
// 256 x 256 tile does a third more work per workgroup and is taken only
// when it needs clearly fewer waves than 128 x 384, and 192 x 256 when it
// streams fewer rows in all (one wave of 228 workgroups at 512 rows).
// Measured on MI355X with weights out of cache (4B shape, SwiGLU epilogue):
// 512 rows 63-72 us (128 x 384) against 69-72 us for the LDS-staged
// 256 x 192 tiles; 768 rows 78 us (256 x 256) against 122 us; 16,925 rows
// 1,473 us against 1,659 us for the LDS-staged 256 x 256 tiles; 27B shape at
// 1,024 rows 359 us (128 x 384) against 435 us.
int gate_up_direct(const Model* m, const LayerW& L, int T) {
  if (!L.w_gu_frag || T <= 0 || m->cfg.ffn % 8) return 0;   // SwiGLU rows written in 16-byte chunks
  auto waves = [&](int t) { return (gemm_wd_tiles(t, T, L.n_gu) + m->n_cu - 1) / m->n_cu; };
  const long long w1 = waves(1), w2 = waves(2), w3 = waves(3);
  const int t = 11 * w2 < 10 * w1 ? 2 : 1;
  return w3 * gemm_wd_panel(3) < (t == 2 ? w2 : w1) * gemm_wd_panel(t) ? 3 : t;
}

// Of the weight-direct tiles given (earlier ones preferred on ties), the one
// with the fewest waves of workgroups times operand rows per K step: the
// operand stream into each CU bounds these launches, and a last wave that
// leaves CUs idle costs a whole wave.  16,925 rows: 224 x 256 tiles take the
// d-wide down projection in 2.97 waves where 256 x 256 take 2.62, rounded up
// to 3 (1,440 against 1,536 rows per K step), and the attention QKV in 3.6
// against 3.1 (4 waves either way, 480 against 512 rows).
int wd_pick(const Model* m, int T, int N, std::initializer_list<int> tiles) {
  int best = 0;
  long long cost = LLONG_MAX;
  for (int t : tiles) {
    const long long c = (gemm_wd_tiles(t, T, N) + m->n_cu - 1) / m->n_cu * gemm_wd_panel(t);
    if (c < cost) {
      cost = c;
      best = t;
    }
  }
  return best;
}

// The down projection on the weight-direct kernel (256 x 256 or 224 x 256
// tiles) when it runs without a K split and its tiles fill the chip at least
// once: the weights bypass LDS as in the gate/up GEMM (4B shape, 16,925
// rows, on MI355X: 930 -> 817 us; the out-projection, K = 2,048, gained
// nothing: 270 against 275 us).  Same K order as the LDS kernels, so rows
// stay bitwise independent of M.  0: not on the weight-direct kernel.
int residual_direct(const Model* m, const void* frag, int T, int split) {
  if (!frag || split != 1 || gemm_wd_tiles(2, T, m->cfg.d_model) < m->n_cu) return 0;
  return wd_pick(m, T, m->cfg.d_model, {2, 4});
}

// The mixer in-projections (linear-attention q|k|v|gate, attention q|k|v)
// on the weight-direct kernel's 256 x 256 or 224 x 256 tiles when those fill
// the chip, with the staged bf16 epilogue.  Same K order as the LDS kernels.
int in_direct(const Model* m, const LayerW& L, int T) {
  if (!L.w_in_frag || gemm_wd_tiles(2, T, L.n_in) < m->n_cu) return 0;
  return wd_pick(m, T, L.n_in, {2, 4});
}

// Largest K split the workspace allows for an M-row GEMM with a d-wide
// output (the GEMM picks the split it uses, up to this).
int max_split(const Model* m, const Plan* p, int M) {
  if (p->invariant) return 1;     // the K order of a row must not depend on M
  return M <= m->split_max_rows ? 4 : 1;
}

// GEMM configuration: chosen by shape, except that the row-invariant mode
// keeps fp32 GEMMs on the one configuration whose K order does not depend on
// the number of rows (bf16 configurations all share one K order).
int gemm_cfg(const Model* m, const Plan* p) { return p->invariant && !m->bf16 ? 0 : GEMM_AUTO; }

int run_pass(Model* m, Plan* p, const PassPlan& ps, bool xn_first, hipStream_t s) {
  const s1_config& c = m->cfg;
  const int d = c.d_model, H = c.la_heads, dk = c.la_dk, dv = c.la_dv;
  const int Hq = c.fa_q_heads, Hkv = c.fa_kv_heads, hd = c.fa_head_dim;
  const int T = ps.T, r0 = ps.r0;
  if (T == 0) return S1_OK;
  const size_t es = m->esz;
  char* xn = static_cast<char*>(m->xn) + (size_t)r0 * d * es;
  float* x = m->x + (size_t)r0 * d;
  char* qkv = static_cast<char*>(m->qkv);
  char* att = static_cast<char*>(m->att);
  const long long kvld = (long long)Hkv * hd;
  bool xn_ready = xn_first;   // xn already holds this layer's normalised input
  // the deferred norm (gains folded into the consuming weights): xn holds
  // either the normalised rows without the gain (from a kernel that had
  // whole rows: the embedding gather, a K split's reduction, a norm pass) or,
  // after a residual GEMM without a K split, the rows themselves, which the
  // consuming GEMM scales by rstd (xn_scaled)
  bool xn_scaled = false;
  float* rstd = m->fold ? m->rstd + r0 : nullptr;
  auto defer_norm = [&](GemmArgs& a) {
    a.rs_out = rstd;
    a.ss_parts = m->ssq + r0;
    a.ss_ld = m->ss_ld;
    a.tickets = m->tickets;
  };
  auto norm_pass = [&](const float* gain) {   // a norm that no GEMM epilogue produced
    return launch_rmsnorm(m->bf16, x, m->fold ? nullptr : gain, xn, T, d, c.rms_eps, s, rstd);
  };
  for (int l = 0; l < c.n_layers; ++l) {
    const LayerW& L = m->layers[l];
    if (ps.n_inj) {   // replaced layer inputs: the rows, then their norm
      S1_TRY(launch_gather_rows(p->inj_src + (size_t)l * p->n_inj * d, d, ps.inj_idx, ps.inj_rows, ps.n_inj,
                                m->x, s),
             "layer inputs");
      xn_ready = false;
    }
    if (!xn_ready) {
      S1_TRY(norm_pass(L.attn_norm), "rmsnorm");
      MARK(KC_RMSNORM);
      xn_scaled = false;
    }
    GemmArgs g{};
    g.A = xn;
    g.row_scale = xn_scaled ? rstd : nullptr;
    g.M = T;
    g.K = d;
    g.lda = d;
    g.ldw = d;
    g.W = L.w_in;
    g.N = L.n_in;
    if (!L.full) {
      g.out0 = qkv + (size_t)r0 * m->ld_qkv * es;
      g.ld0 = m->ld_qkv;
      g.out1 = m->lg + (size_t)r0 * H;
      g.ld1 = H;
      g.nsplit = 2 * H * dk + H * dv;
      const bool gdn = c.la_kind == S1_LA_GDN;
      if (gdn) {
        g.out2 = m->beta + (size_t)r0 * H;
        g.nsplit2 = g.nsplit + H;
      }
      if (const int wt = in_direct(m, L, T); wt && gemm_wd_ok(EPI_GATE, g)) {
        g.W = L.w_in_frag;
        S1_TRY(launch_gemm_wd(EPI_GATE, g, wt, s), "linear-attention in-projection");
      } else {
        S1_TRY(launch_gemm(m->bf16, EPI_GATE, g, 1, nullptr, s, gemm_cfg(m, p)), "linear-attention in-projection");
      }
      MARK(KC_GEMM_LA_IN);
      float* states = m->states + (size_t)L.la_idx * c.max_prefixes * H * dk * dv;
      if (gdn) {
        char* q2 = static_cast<char*>(m->qkv2);
        const size_t Cc = (size_t)2 * H * dk + (size_t)H * dv;
        char* hist = static_cast<char*>(m->conv_hist) + (size_t)L.la_idx * c.max_prefixes * 3 * Cc * es;
        S1_TRY(launch_gdn_conv(qkv, q2, m->ld_qkv, L.conv, H, r0, T, ps.row_seq, ps.gseqs, hist,
                               1.f / sqrtf((float)dk), s),
               "Gated DeltaNet convolution");
        S1_TRY(launch_gdn_scan(q2, q2 + (size_t)H * dk * es, q2 + (size_t)2 * H * dk * es, m->ld_qkv, m->lg,
                               m->beta, H, att, m->ld_att, ps.chunks, ps.n_chunks, ps.gseqs, ps.n_seqs, states, H,
                               m->gdn_ws, s),
               "Gated DeltaNet scan");
      } else if (ps.chunked || (p->invariant && ps.n_chunks > 0))
        S1_TRY(launch_scan_chunked(qkv, qkv + (size_t)H * dk * es, qkv + (size_t)2 * H * dk * es, m->ld_qkv,
                                   m->lg, H, att, m->ld_att, ps.chunks, ps.n_chunks, ps.cseqs, ps.n_seqs,
                                   m->cstates, m->gamma, states, H, s, ps.max_nc),
               "linear-attention scan (chunk-parallel)");
      else
        S1_TRY(launch_scan(m->bf16, qkv, qkv + (size_t)H * dk * es, qkv + (size_t)2 * H * dk * es,
                           m->ld_qkv, m->lg, H, att, m->ld_att, ps.scan, ps.n_seqs, states, H, dk, dv, s,
                           p->invariant ? INT_MAX : ps.max_len),   // one fp32 schedule in the row-invariant mode
               "linear-attention scan");
      MARK(KC_LA_SCAN);
    } else {
      char* kc = static_cast<char*>(m->kc) + (size_t)L.fa_idx * c.max_tokens * kvld * es;
      char* vc = static_cast<char*>(m->vc) + (size_t)L.fa_idx * c.max_tokens * kvld * es;
      g.out0 = qkv + (size_t)r0 * m->ld_qkv * es;
      g.ld0 = m->ld_qkv;
      g.out1 = kc + (size_t)r0 * kvld * es;
      g.ld1 = (int)kvld;
      g.out2 = vc + (size_t)r0 * kvld * es;
      g.ld2 = (int)kvld;
      g.nsplit = Hq * hd;
      g.nsplit2 = (Hq + Hkv) * hd;
      g.head_dim = hd;
      g.pos = p->pos + r0;
      g.rope = m->rope;
      if (const int wt = in_direct(m, L, T); wt && gemm_wd_ok(EPI_QKV, g)) {
        g.W = L.w_in_frag;
        S1_TRY(launch_gemm_wd(EPI_QKV, g, wt, s), "attention QKV projection");
      } else {
        S1_TRY(launch_gemm(m->bf16, EPI_QKV, g, 1, nullptr, s, gemm_cfg(m, p)), "attention QKV projection");
      }
      MARK(KC_GEMM_FA_QKV);
      const bool split = !p->invariant;
      S1_TRY(launch_attention(m->bf16, qkv, m->ld_qkv, kc, vc, (int)kvld, att, m->ld_att, ps.attn,
                              split ? ps.blocks : ps.blocks_inv, split ? ps.n_blocks : ps.n_blocks_inv, Hq, Hkv,
                              hd, ps.attn_rows, ps.attn_part, s),
             "attention");
      if (split && ps.n_comb)
        S1_TRY(launch_attn_combine(ps.comb_rows, ps.n_comb, ps.attn_part, att, m->ld_att, Hq, s),
               "attention combine");
      MARK(KC_ATTENTION);
    }
    GemmArgs go{};
    go.A = att + (size_t)r0 * m->ld_att * es;
    go.lda = m->ld_att;
    go.W = L.w_o;
    go.ldw = L.k_o;
    go.M = T;
    go.N = d;
    go.K = L.k_o;
    go.out0 = x;
    go.ld0 = d;
    go.norm_w = m->fold ? nullptr : L.ffn_norm;
    go.norm_out = xn;
    go.norm_eps = c.rms_eps;
    if (m->fold) defer_norm(go);
    int normed = NORM_NONE;
    if (const int wt = residual_direct(m, L.w_o_frag, T, max_split(m, p, T)); wt == 4) {
      // only on the 224 x 256 tiles: at K = 2,048 the 256 x 256 weight-direct
      // tiles gained nothing over the LDS-staged ones
      go.W = L.w_o_frag;
      S1_TRY(launch_gemm_wd(EPI_RESID, go, wt, s), "mixer out-projection");
      normed = go.rs_out ? NORM_DEFERRED : NORM_NONE;
    } else {
      S1_TRY(launch_gemm(m->bf16, EPI_RESID, go, max_split(m, p, T), m->splitws, s, gemm_cfg(m, p), &normed),
             "mixer out-projection");
    }
    MARK(KC_GEMM_O);
    if (normed == NORM_NONE) {
      S1_TRY(norm_pass(L.ffn_norm), "rmsnorm");
      MARK(KC_RMSNORM);
    }
    GemmArgs gu{};
    gu.A = xn;
    gu.row_scale = normed == NORM_DEFERRED ? rstd : nullptr;
    gu.lda = d;
    gu.W = L.w_gu;
    gu.ldw = d;
    gu.M = T;
    gu.N = L.n_gu;
    gu.K = d;
    gu.out0 = static_cast<char*>(m->hbuf) + (size_t)r0 * c.ffn * es;
    gu.ld0 = c.ffn;
    gu.n_valid = c.ffn;
    if (const int wd = gate_up_direct(m, L, T)) {
      gu.W = L.w_gu_frag;
      S1_TRY(launch_gemm_wd(EPI_SWIGLU, gu, wd, s), "FFN gate/up");
    } else {
      S1_TRY(launch_gemm(m->bf16, EPI_SWIGLU, gu, 1, nullptr, s, gemm_cfg(m, p)), "FFN gate/up");
    }
    MARK(KC_GEMM_GATE_UP);
    GemmArgs gd{};
    gd.A = gu.out0;
    gd.lda = c.ffn;
    gd.W = L.w_down;
    gd.ldw = c.ffn;
    gd.M = T;
    gd.N = d;
    gd.K = c.ffn;
    gd.out0 = x;
    gd.ld0 = d;
    // the next layer's input norm: fused into the K split's reduction, or
    // deferred (its statistics from this GEMM's epilogue)
    if (l + 1 < c.n_layers) {
      gd.norm_w = m->fold ? nullptr : m->layers[l + 1].attn_norm;
      gd.norm_out = xn;
      gd.norm_eps = c.rms_eps;
      if (m->fold) defer_norm(gd);
    }
    if (const int wt = residual_direct(m, L.w_down_frag, T, max_split(m, p, T))) {
      gd.W = L.w_down_frag;
      S1_TRY(launch_gemm_wd(EPI_RESID, gd, wt, s), "FFN down");
      xn_ready = xn_scaled = gd.rs_out != nullptr;   // without a K split: the rows and their scales
    } else {
      int nd = NORM_NONE;
      S1_TRY(launch_gemm(m->bf16, EPI_RESID, gd, max_split(m, p, T), m->splitws, s, gemm_cfg(m, p), &nd),
             "FFN down");
      xn_ready = nd != NORM_NONE;
      xn_scaled = nd == NORM_DEFERRED;
    }
    MARK(KC_GEMM_DOWN);
    if (ps.n_cap) {
      S1_TRY(launch_gather_rows(m->x, d, ps.cap_rows, ps.cap_dst, ps.n_cap,
                                p->cap_out + (size_t)(l + 1) * p->n_cap * d, s),
             "capture");
      MARK(KC_CAPTURE);
    }
  }
  return S1_OK;
}

}  // namespace

int run_plan(Model* m, Plan* p, float* d_probs, void* d_dec, hipStream_t s) {
  const s1_config& c = m->cfg;
  if (p->T == 0) return S1_OK;
  if (m->prof) m->prof->begin(s);
  // the gather writes the first layer's normalised input too when the row fits the fused kernel
  const bool fused = c.n_layers > 0 && c.d_model % 4 == 0 && c.d_model <= 16384;
  if (fused)
    S1_TRY(launch_embed_norm(m->bf16, p->ids, m->embed, m->x, p->T, c.d_model,
                             m->fold ? nullptr : m->layers[0].attn_norm, m->xn, c.rms_eps, s,
                             m->fold ? m->rstd : nullptr),
           "embedding and first norm");
  else
    S1_TRY(launch_embed(m->bf16, p->ids, m->embed, m->x, p->T, c.d_model, s), "embedding");
  MARK(KC_EMBED);
  for (int ps = 0; ps < p->n_passes; ++ps)
    if (p->pass[ps].n_cap)
      S1_TRY(launch_gather_rows(m->x, c.d_model, p->pass[ps].cap_rows, p->pass[ps].cap_dst,
                                p->pass[ps].n_cap, p->cap_out, s),
             "capture");
  for (int ps = 0; ps < p->n_passes; ++ps) {
    const int rc = run_pass(m, p, p->pass[ps], fused, s);
    if (rc) return rc;
  }
  if (p->Q > 0)
    S1_TRY(launch_readout(m->bf16, m->x, c.d_model, m->final_norm, c.rms_eps, m->embed, p->Q, p->q_row,
                          p->opt_off, p->opt_ids, p->q_type, d_probs, d_dec, p->max_k, s),
           "readout");
  if (p->Q > 0) MARK(KC_READOUT);
  if (p->feat.n_targets > 0) {
    S1_TRY(launch_feat_norm(m->bf16, m->x, c.d_model, p->feat.rows, p->feat.R, m->final_norm, c.rms_eps,
                            c.vocab, p->feat_ws, s),
           "feature rows");
    MARK(KC_FEATURES);
    S1_TRY(launch_vocab_lse(m->bf16, m->embed, c.vocab, c.d_model, p->feat.R, p->feat_ws, s), "vocabulary lse");
    MARK(KC_VOCAB_LSE);
    S1_TRY(launch_lse_merge(m->bf16, c.vocab, c.d_model, p->feat.R, p->feat_ws, s), "lse merge");
    S1_TRY(launch_feat_targets(m->bf16, c.d_model, m->embed, c.vocab, p->feat, p->feat_logp, p->feat_cand_lp,
                               p->feat_cand_norm, p->feat_ws, s),
           "feature targets");
    MARK(KC_FEATURES);
  }
  return S1_OK;
}

}  // namespace s1

namespace s1 {

// Capture the forward of a plan into a HIP graph on stream s (it must not be
// the null stream) and replay it.  Only kernel launches are recorded.
int run_plan_graph(Model* m, Plan* p, float* d_probs, void* d_dec, hipStream_t s) {
  if (p->gexec && (p->g_probs != d_probs || p->g_dec != d_dec || p->g_cap != p->cap_out || p->g_inj != p->inj_src))
    p->drop_graph();
  if (!p->gexec) {
    hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) return set_error(S1_EDEVICE, hip_msg(e, "begin graph capture"));
    const int rc = run_plan(m, p, d_probs, d_dec, s);
    hipGraph_t g = nullptr;
    e = hipStreamEndCapture(s, &g);
    if (rc) {
      if (g) (void)hipGraphDestroy(g);
      return rc;
    }
    if (e != hipSuccess) return set_error(S1_EDEVICE, hip_msg(e, "end graph capture"));
    hipGraphExec_t x = nullptr;
    e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
    if (e != hipSuccess) {
      (void)hipGraphDestroy(g);
      return set_error(S1_EDEVICE, hip_msg(e, "instantiate graph"));
    }
    p->graph = g;
    p->gexec = x;
    p->g_probs = d_probs;
    p->g_dec = d_dec;
    p->g_cap = p->cap_out;
    p->g_inj = p->inj_src;
  }
  const hipError_t e = hipGraphLaunch(p->gexec, s);
  if (e != hipSuccess) return set_error(S1_EDEVICE, hip_msg(e, "graph launch"));
  return S1_OK;
}

}  // namespace s1
