// Host-side fuzz of the library's validation and launch planning, built
// with AddressSanitizer and UndefinedBehaviorSanitizer on the host code only
// (test_host_sanitizers_cpu.py; no GPU needed, nothing is launched).
// Requests are random but honour the calling contract: every array holds
// the number of elements its counts declare, so any out-of-bounds access,
// overflow or undefined shift the sanitizers report is the library's.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "../include/s1.h"
#include "../include/s1_kernels.h"

namespace {

std::mt19937 rng;
int pick(int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); }

s1_config tiny_config() {
  s1_config c{};
  c.n_layers = 2; c.full_every = 2; c.d_model = 256; c.ffn = 688; c.vocab = 4096;
  c.la_heads = 4; c.la_dk = 64; c.la_dv = 64; c.fa_q_heads = 4; c.fa_kv_heads = 4; c.fa_head_dim = 64;
  c.rope_base = 10000.f; c.rms_eps = 1e-6f; c.lora_rank = 8; c.lora_alpha = 16.f; c.lora_targets = 0xF;
  c.dtype = S1_F32; c.max_tokens = pick(1, 2000); c.max_seqs = pick(1, 12); c.max_questions = pick(1, 16);
  c.max_options = pick(2, 12); c.max_prefixes = pick(1, 3); c.max_positions = pick(1, 4000); c.la_kind = S1_LA_GLA;
  return c;
}

int fuzz_batch(const s1_config& c) {
  const int n = pick(0, 8);
  std::vector<int32_t> cu(n + 1, 0);
  for (int i = 1; i <= n; ++i) cu[i] = cu[i - 1] + (pick(0, 9) == 0 ? -pick(1, 5) : pick(0, 300));
  if (pick(0, 9) == 0 && n > 0) cu[0] = pick(-3, 3);
  int tmax = 0;
  for (int x : cu) tmax = std::max(tmax, x);
  std::vector<int32_t> ids(std::max(tmax, 1));
  for (auto& t : ids) t = pick(0, 30) == 0 ? pick(-2, c.vocab + 2) : pick(0, c.vocab - 1);
  std::vector<int32_t> pre(std::max(n, 1), -1);
  for (int i = 0; i < n; ++i)
    if (pick(0, 3) == 0) pre[i] = pick(-2, n);
  const int Q = pick(0, 10);
  std::vector<int32_t> qs(std::max(Q, 1)), qm(std::max(Q, 1)), off(Q + 1, 0);
  std::vector<uint8_t> qt(std::max(Q, 1));
  for (int j = 0; j < Q; ++j) {
    qs[j] = pick(-1, n);
    qm[j] = pick(-1, 310);
    qt[j] = (uint8_t)pick(0, 3);
    off[j + 1] = off[j] + (pick(0, 9) == 0 ? pick(-3, 1) : pick(2, 7));
  }
  int omax = 0;
  for (int x : off) omax = std::max(omax, x);
  std::vector<int32_t> opt(std::max(omax, 1));
  for (auto& o : opt) o = pick(0, 40) == 0 ? pick(-1, c.vocab) : pick(0, c.vocab - 1);
  s1_batch b{n, cu.data(), ids.data(), pick(0, 1) ? pre.data() : nullptr, Q, qs.data(), qm.data(), qt.data(),
             off.data(), opt.data()};
  const int rc = s1_validate(&c, &b);
  if (rc != S1_OK && rc != S1_EINVAL && rc != S1_EBUDGET) {
    std::fprintf(stderr, "unexpected status %d\n", rc);
    std::exit(2);
  }
  if (rc == S1_OK && n > 0) {
    // the attention plan of the batch's sequences as the decoder lays them out
    std::vector<int32_t> r0(n), len(n), pr0(n), plen(n);
    for (int i = 0; i < n; ++i) {
      r0[i] = cu[i];
      len[i] = cu[i + 1] - cu[i];
      const int p = b.prefix_of ? b.prefix_of[i] : -1;
      pr0[i] = p >= 0 ? cu[p] : 0;
      plen[i] = p >= 0 ? cu[p + 1] - cu[p] : 0;
    }
    const int rows = cu[n] + 1;
    std::vector<int32_t> blocks(5 * (4096 + 64 * rows)), shared(5 * n), row_np(rows);
    int32_t nb = 0, ns = 0, pc = 0;
    const int piece = pick(0, 3) == 0 ? 0 : (pick(0, 1) ? -1 : 64 * pick(1, 8));
    const int prc = s1k_attention_plan(n, r0.data(), len.data(), r0.data(), pr0.data(), plen.data(), 16,
                                       32 << pick(0, 2), piece, pick(1, 512), 4096 + 64 * rows, blocks.data(), &nb,
                                       n, shared.data(), &ns, rows, row_np.data(), &pc);
    if (prc != S1_OK && prc != S1_EINVAL) {
      std::fprintf(stderr, "unexpected plan status %d\n", prc);
      std::exit(2);
    }
  }
  return rc;
}

}  // namespace

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 20000;
  rng.seed(argc > 2 ? (unsigned)std::atoi(argv[2]) : 1u);
  int counts[5] = {0};
  for (int it = 0; it < iters; ++it) {
    const s1_config c = tiny_config();
    const int rc = fuzz_batch(c);
    counts[-rc]++;
  }
  // malformed configs
  for (int it = 0; it < 2000; ++it) {
    s1_config c = tiny_config();
    int32_t* f = reinterpret_cast<int32_t*>(&c);
    f[pick(0, 10)] = pick(-3, 300);
    (void)s1_validate(&c, nullptr);
  }
  std::printf("ok %d %d %d\n", counts[0], counts[1], counts[4]);
  return 0;
}
