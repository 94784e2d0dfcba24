// Exercises the host side of every C entry point (argument checks, the split
// and schedule planners, the RoPE table) under the host sanitizers, with the
// kernel launchers replaced by counting stand-ins.  Device pointers are fake,
// aligned addresses that only a launcher would dereference.  Exits 1 on the
// first unexpected status; the sanitizers abort on any memory error or
// undefined behaviour.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "mla.h"
#include "mla_internal.h"

extern int g_launches;

namespace {

int failures = 0;
#define FAIL(msg, ...) (std::printf("line %d: " msg "\n", __LINE__, ##__VA_ARGS__), ++failures)
void* const F = reinterpret_cast<void*>(uintptr_t(0x10000));
void* const MIS = reinterpret_cast<void*>(uintptr_t(0x10008));
float* const FF = static_cast<float*>(F);
int32_t* const FI = static_cast<int32_t*>(F);

void expect(int32_t got, int32_t want, const char* what, int line) {
  if (got != want) {
    std::printf("line %d: %s returned %d, expected %d\n", line, what, got, want);
    ++failures;
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

void plan_invariants(std::mt19937& rng) {
  for (int iter = 0; iter < 300; ++iter) {
    const int B = int(rng() % 9);
    const int q_len = 1 + int(rng() % 5);
    const int n_h = (rng() % 2) ? 128 : 16;
    const int slots = 1 + int(rng() % 300);
    std::vector<int32_t> lens(B);
    for (auto& L : lens) L = (rng() % 4 == 0) ? int(rng() % 3) : int(rng() % 5000);
    int32_t n_work = 0, n_lists = 0, n_split = 0, n_parts = 0;
    std::vector<int32_t> lists(slots + 1);
    // sizing call: max_work 0 reports the size needed
    int32_t st = mla_plan_decode(lens.data(), B, q_len, 64, n_h, slots, 0, nullptr, &n_work,
                                 lists.data(), &n_lists, nullptr, &n_split, &n_parts);
    if (st != MLA_OK && st != MLA_ERR_SHAPE) { FAIL("sizing status %d", st); continue; }
    const int max_work = n_work > 0 ? n_work : 1;
    std::vector<int32_t> work(4 * max_work), split(3 * max_work);
    st = mla_plan_decode(lens.data(), B, q_len, 64, n_h, slots, max_work, work.data(), &n_work,
                         lists.data(), &n_lists, split.data(), &n_split, &n_parts);
    if (st != MLA_OK) { FAIL("plan status %d", st); continue; }
    if (n_lists < 1 || n_lists > slots || lists[0] != 0 || lists[n_lists] != n_work)
      FAIL("lists: n_lists %d slots %d first %d last %d n_work %d", n_lists, slots, lists[0],
           lists[n_lists], n_work);
    for (int k = 0; k < n_lists; ++k)
      if (lists[k] > lists[k + 1]) FAIL("lists not ordered");
    for (int i = 0; i < n_work; ++i) {
      const int32_t row = work[4 * i], kb = work[4 * i + 1], ke = work[4 * i + 2],
                    slot = work[4 * i + 3];
      if (row < 0 || row >= B * q_len || kb > ke || slot >= n_parts || slot < -1)
        FAIL("work item %d: row %d keys [%d, %d) slot %d of %d", i, row, kb, ke, slot, n_parts);
    }
    for (int j = 0; j < n_split; ++j)
      if (split[3 * j + 1] < 0 || split[3 * j + 1] + split[3 * j + 2] > n_parts)
        FAIL("split entry %d", j);
  }
}

void split_plan_partitions(std::mt19937& rng) {
  for (int iter = 0; iter < 200; ++iter) {
    const int B = 1 + int(rng() % 6), S = 1 + int(rng() % 70);
    std::vector<int32_t> lens(B), be(2 * B * S);
    for (auto& L : lens) L = int(rng() % 9000);
    EXPECT(mla_split_plan(lens.data(), B, 64, S, be.data()), MLA_OK);
    for (int b = 0; b < B; ++b) {
      int32_t prev = 0;
      for (int s = 0; s < S; ++s) {
        const int32_t lo = be[2 * (b * S + s)], hi = be[2 * (b * S + s) + 1];
        if (lo != prev || hi < lo) FAIL("split %d of row %d: [%d, %d) after %d", s, b, lo, hi, prev);
        prev = hi;
      }
      if (prev != lens[b]) FAIL("splits of row %d end at %d, not %d", b, prev, lens[b]);
    }
  }
  std::vector<int32_t> bad = {5, -1}, be(4);
  EXPECT(mla_split_plan(bad.data(), 2, 64, 1, be.data()), MLA_ERR_SHAPE);
}

void rope_table() {
  double th[32];
  EXPECT(mla_rope_theta(1e4, 40, 1, 32, 4096, th), MLA_OK);
  if (!(th[0] == 1.0 && std::fabs(th[31] * 40 - std::pow(1e4, -62.0 / 64)) < 1e-18)) ++failures;
  EXPECT(mla_rope_theta(1e4, 40, 1, 32, 4096, nullptr), MLA_ERR_NULL);
  EXPECT(mla_rope_theta(1e4, 0.5, 1, 32, 4096, th), MLA_ERR_SHAPE);
  EXPECT(mla_rope_theta(NAN, 40, 1, 32, 4096, th), MLA_ERR_SHAPE);
}

void entry_points() {
  double good[32], bad[32];
  for (int k = 0; k < 32; ++k) { good[k] = 0.5; bad[k] = k == 9 ? -1.0 : 0.5; }
  const int before = g_launches;
  EXPECT(mla_kv_append(F, 1, 4, 64, FI, 1, 4, F, F, FI, FI, 3, 1e4, nullptr, nullptr), MLA_OK);
  EXPECT(mla_kv_append(F, 1, 4, 64, FI, 1, 4, F, F, FI, FI, 3, 1e4, bad, nullptr), MLA_ERR_SHAPE);
  EXPECT(mla_kv_append(MIS, 1, 4, 64, FI, 1, 4, F, F, FI, FI, 3, 1e4, good, nullptr), MLA_ERR_ALIGN);
  EXPECT(mla_kv_append_fp8(F, FF, 1, 4, 64, FI, 1, 4, F, F, FI, FI, 3, 1e4, good, nullptr), MLA_OK);
  EXPECT(mla_kv_append_fp8(F, nullptr, 1, 4, 64, FI, 1, 4, F, F, FI, FI, 3, 1e4, good, nullptr),
         MLA_ERR_NULL);
  EXPECT(mla_absorb_q(F, F, F, FI, 4, 16, 1, 1e4, good, F, nullptr), MLA_OK);
  EXPECT(mla_absorb_q(F, F, F, FI, 4, 24, 1, 1e4, nullptr, F, nullptr), MLA_ERR_SHAPE);
  EXPECT(mla_append_absorb_q(F, 4, 64, FI, 1, 4, F, F, FI, FI, 3, F, F, F, FI, 4, 16, 1, 1e4,
                             nullptr, F, nullptr), MLA_OK);
  EXPECT(mla_append_absorb_q(F, 4, 64, FI, 1, 4, F, F, FI, FI, 0, F, F, F, FI, 4, 16, 1, 1e4,
                             good, F, nullptr), MLA_OK);
  EXPECT(mla_append_absorb_q(nullptr, 4, 64, FI, 1, 4, F, F, FI, FI, 0, F, F, F, FI, 4, 16, 1,
                             1e4, good, F, nullptr), MLA_OK);
  EXPECT(mla_append_absorb_q(MIS, 4, 64, FI, 1, 4, F, F, FI, FI, 3, F, F, F, FI, 4, 16, 1, 1e4,
                             good, F, nullptr), MLA_ERR_ALIGN);
  EXPECT(mla_append_absorb_q(F, 4, 32, FI, 1, 4, F, F, FI, FI, 3, F, F, F, FI, 4, 16, 1, 1e4,
                             good, F, nullptr), MLA_ERR_SHAPE);
  EXPECT(mla_append_absorb_q(F, 4, 64, FI, 1, 4, F, F, FI, FI, 3, F, F, F, FI, 4, 24, 1, 1e4,
                             good, F, nullptr), MLA_ERR_SHAPE);
  EXPECT(mla_append_absorb_q(F, 4, 64, FI, 1, 4, F, F, FI, FI, 3, F, F, F, FI, 0, 24, 1, 1e4,
                             good, F, nullptr), MLA_OK);
  EXPECT(mla_append_absorb_q(F, 4, 64, FI, 1, 4, F, F, FI, FI, 3, nullptr, F, F, FI, 4, 16, 1,
                             1e4, good, F, nullptr), MLA_ERR_NULL);
  EXPECT(mla_append_absorb_q(F, 4, 64, FI, 1, 4, F, F, FI, FI, 3, F, F, F, FI, 4, 16, 7, 1e4,
                             good, F, nullptr), MLA_ERR_DTYPE);
  EXPECT(mla_append_absorb_q(F, 4, 64, FI, 1, 4, F, F, FI, FI, 3, F, F, F, FI, 4, 16, 1, 1e4,
                             bad, F, nullptr), MLA_ERR_SHAPE);
  EXPECT(mla_decode_paged(F, F, 4, 64, FI, 4, FI, 2, 1, 128, 1, 0.07f, 3, FF, FF, FF, FF, nullptr),
         MLA_OK);
  EXPECT(mla_decode_paged(F, F, 4, 64, FI, 4, FI, 2, 1, 48, 1, 0.07f, 1, FF, FF, FF, FF, nullptr),
         MLA_ERR_SHAPE);
  EXPECT(mla_decode_paged_fp8(F, F, FF, 4, 64, FI, 4, FI, 2, 1, 16, 0.07f, 1, nullptr, nullptr, FF,
                              FF, nullptr), MLA_OK);
  EXPECT(mla_decode_paged_planned(F, F, 4, 64, FI, 4, 2, 1, 64, 1, 0.07f, FI, 5, FI, 2, FF, FF, 3,
                                  FF, FF, nullptr), MLA_OK);
  EXPECT(mla_decode_paged_planned_fp8(F, F, FF, 4, 64, FI, 4, 2, 1, 32, 0.07f, FI, 5, nullptr, 0,
                                      FF, FF, 3, FF, FF, nullptr), MLA_OK);
  EXPECT(mla_decode_paged_planned_fp8(F, F, FF, 4, 64, FI, 4, 2, 1, 128, 0.07f, FI, 5, FI, 0,
                                      FF, FF, 3, FF, FF, nullptr), MLA_ERR_SHAPE);
  EXPECT(mla_splitkv_combine(FF, FF, 2, 3, 1, 16, FF, FF, nullptr), MLA_OK);
  EXPECT(mla_combine_planned(FF, FF, FI, 2, 16, FF, FF, nullptr), MLA_OK);
  EXPECT(mla_out_proj(FF, F, 4, 16, 1, FF, nullptr), MLA_OK);
  EXPECT(mla_out_proj_planned(FF, FF, FF, FI, 2, F, 4, 16, 1, FF, FF, nullptr), MLA_OK);
  const int64_t kw = mla_kv_produce_workspace(4, 64);
  EXPECT(mla_kv_produce(F, F, FF, F, 4, 64, 1, 1e-6f, 1e4f, good, F, 4, 64, FI, 1, 4, FI, FI, F,
                        kw, nullptr), MLA_OK);
  EXPECT(mla_kv_produce(F, F, FF, F, 4, 64, 1, 1e-6f, 1e4f, good, F, 4, 64, FI, 1, 4, FI, FI, F,
                        kw - 1, nullptr), MLA_ERR_SHAPE);
  const int64_t qw = mla_q_produce_workspace(4, 64, 64, 1);
  EXPECT(mla_q_produce(F, F, FF, F, F, 4, 64, 64, 2, 1, 1e-6f, F, F, F, qw, nullptr), MLA_OK);
  EXPECT(mla_q_produce_direct(F, F, F, 4, 64, 2, 1, F, F, nullptr), MLA_OK);
  const int64_t ow = mla_o_proj_workspace(4, 2, 64, 1);
  EXPECT(mla_o_proj(FF, F, 4, 2, 64, 1, F, F, ow, nullptr), MLA_OK);
  std::vector<int32_t> lens = {300, 200};
  const int64_t pw = mla_prefill_mha_workspace(300, 16);
  EXPECT(mla_prefill_mha(F, F, FI, F, F, F, 16, 64, FI, 8, lens.data(), 2, 100, 16, 1, 0.07f, 1e4f,
                         good, FF, FF, F, pw, nullptr), MLA_OK);
  EXPECT(mla_prefill_mha(F, F, FI, F, F, F, 16, 64, FI, 4, lens.data(), 2, 100, 16, 1, 0.07f, 1e4f,
                         nullptr, FF, FF, F, pw, nullptr), MLA_ERR_SHAPE);
  for (int s = -1; s < 9; ++s)
    if (mla_status_string(s) == nullptr) ++failures;
  if (mla_abi_version() != MLA_ABI_VERSION) ++failures;
  // arming stores the handles for this thread; the next launch takes them
  int ev0 = 0, ev1 = 0;
  EXPECT(mla_time_attention(&ev0, &ev1), MLA_OK);
  const mla::KernelEvents armed = mla::take_attention_events();
  if (armed.start != (hipEvent_t)&ev0 || armed.stop != (hipEvent_t)&ev1) ++failures;
  const mla::KernelEvents after = mla::take_attention_events();
  if (after.start != nullptr || after.stop != nullptr) ++failures;
  EXPECT(mla_time_attention(nullptr, nullptr), MLA_OK);
  if (g_launches - before < 16) {
    std::printf("only %d launches reached the stand-ins\n", g_launches - before);
    ++failures;
  }
}

}  // namespace

int main() {
  std::mt19937 rng(2024);
  rope_table();
  split_plan_partitions(rng);
  plan_invariants(rng);
  entry_points();
  if (failures) {
    std::printf("%d failures\n", failures);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
