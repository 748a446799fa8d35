// Host-side check of libdecode_attn's C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer: every entry point's argument checks and the
// split planners run on parameter sets that are valid, at the edges of what
// is accepted, and hostile (zeros, negatives, huge sizes and strides, NaN),
// with pointers that are never dereferenced. Built by
// decode_attention_kv_bf16_amd.build.build_host_check() and run by
// tests/test_abi_cpu.py on a machine with no GPU, where every call that
// passes its checks fails at the launch (DA_ERR_HIP) instead of running.
// Exits 0 after printing "host checks passed" when every expected status
// matched; a sanitizer report aborts it.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "decode_attn.h"

// the one HIP runtime call the check makes itself (no HIP headers needed)
extern "C" int hipGetDeviceCount(int* count);
constexpr int hipSuccess = 0;

namespace {

int g_failures = 0;
int g_calls = 0;

void expect(const char* what, int got, int want) {
  ++g_calls;
  if (got != want) {
    ++g_failures;
    fprintf(stderr, "FAIL %s: status %d, expected %d\n", what, got, want);
  }
}

// a status that is not a host-side rejection of valid arguments: OK or the
// launch failing for want of a device
bool launched(int st) { return st == DA_OK || st == DA_ERR_HIP; }

void* const FAKE = reinterpret_cast<void*>(0x10000);      // 16-byte aligned, never dereferenced
void* const FAKE_MIS = reinterpret_cast<void*>(0x10002);  // misaligned
const size_t BIG = size_t(1) << 40;

uint64_t g_rng = 0x9E3779B97F4A7C15ull;
uint64_t next_u64() {
  g_rng ^= g_rng << 13;
  g_rng ^= g_rng >> 7;
  g_rng ^= g_rng << 17;
  return g_rng;
}
// a value from a menu that mixes valid, edge and hostile entries
template <typename T, size_t N>
T pick(const T (&menu)[N]) { return menu[next_u64() % N]; }

da_gqa_params_t gqa(int B = 32, int Hq = 32, int Hkv = 8, int D = 128, int L = 4096) {
  da_gqa_params_t p{};
  p.batch = B; p.num_q_heads = Hq; p.num_kv_heads = Hkv; p.head_dim = D; p.max_seq_len = L;
  p.dtype = DA_DTYPE_BF16; p.softmax_scale = 1.0f / sqrtf((float)D);
  p.q_stride_b = (int64_t)Hq * D; p.q_stride_h = D;
  p.kv_stride_b = (int64_t)L * Hkv * D; p.kv_stride_t = (int64_t)Hkv * D; p.kv_stride_h = D;
  return p;
}

da_mla_params_t mla(int B = 64, int H = 128, int L = 4096) {
  da_mla_params_t p{};
  p.batch = B; p.num_heads = H; p.kv_lora_rank = 512; p.qk_rope_dim = 64; p.qk_nope_dim = 128;
  p.v_head_dim = 128; p.max_seq_len = L; p.softmax_scale = 1.0f / sqrtf(192.f);
  p.cache_stride_b = (int64_t)L * 576; p.cache_stride_t = 576;
  return p;
}

da_paged_kv_t paged(int page_size = 16, int max_blocks = 256, int64_t stride = 16 * 8 * 128) {
  da_paged_kv_t pg{};
  pg.block_table = static_cast<const int32_t*>(FAKE);
  pg.page_size = page_size; pg.max_blocks_per_seq = max_blocks; pg.page_stride = stride;
  return pg;
}

void fixed_cases() {
  // GQA: each rejection of the pages' constraints and of bad layouts
  da_gqa_params_t p = gqa();
  expect("gqa valid", launched(da_gqa_decode(&p, FAKE, FAKE, FAKE, nullptr, (float*)FAKE, nullptr, FAKE, BIG, nullptr)), 1);
  expect("gqa null params", da_gqa_decode(nullptr, FAKE, FAKE, FAKE, nullptr, (float*)FAKE, nullptr, FAKE, BIG, nullptr), DA_ERR_INVALID_ARGUMENT);
  p = gqa(); p.num_kv_heads = 3;
  expect("gqa Hq % Hkv", da_gqa_decode(&p, FAKE, FAKE, FAKE, nullptr, (float*)FAKE, nullptr, FAKE, BIG, nullptr), DA_ERR_INVALID_ARGUMENT);
  p = gqa(); p.head_dim = 96;
  expect("gqa head_dim 96", da_gqa_decode(&p, FAKE, FAKE, FAKE, nullptr, (float*)FAKE, nullptr, FAKE, BIG, nullptr), DA_ERR_UNSUPPORTED);
  p = gqa(); p.kv_stride_t = 1028;
  expect("gqa stride", da_gqa_decode(&p, FAKE, FAKE, FAKE, nullptr, (float*)FAKE, nullptr, FAKE, BIG, nullptr), DA_ERR_INVALID_ARGUMENT);
  p = gqa(); p.softmax_scale = NAN;
  expect("gqa nan scale", da_gqa_decode(&p, FAKE, FAKE, FAKE, nullptr, (float*)FAKE, nullptr, FAKE, BIG, nullptr), DA_ERR_INVALID_ARGUMENT);
  p = gqa(16);
  expect("gqa workspace", da_gqa_decode(&p, FAKE, FAKE, FAKE, nullptr, (float*)FAKE, nullptr, nullptr, 0, nullptr), DA_ERR_WORKSPACE_TOO_SMALL);
  expect("gqa misaligned", da_gqa_decode(&p, FAKE_MIS, FAKE, FAKE, nullptr, (float*)FAKE, nullptr, FAKE, BIG, nullptr), DA_ERR_INVALID_ARGUMENT);
  // MLA
  da_mla_params_t m = mla();
  expect("mla valid", launched(da_mla_decode_absorbed(&m, FAKE, FAKE, FAKE, nullptr, FAKE, FAKE, (float*)FAKE, nullptr, FAKE, BIG, nullptr)), 1);
  m = mla(); m.num_heads = 80;
  expect("mla 80 heads", da_mla_decode_absorbed(&m, FAKE, FAKE, FAKE, nullptr, FAKE, FAKE, (float*)FAKE, nullptr, FAKE, BIG, nullptr), DA_ERR_UNSUPPORTED);
  m = mla(); m.softmax_scale = -1.f;
  expect("mla negative scale", da_mla_decode_absorbed(&m, FAKE, FAKE, FAKE, nullptr, FAKE, FAKE, (float*)FAKE, nullptr, FAKE, BIG, nullptr), DA_ERR_UNSUPPORTED);
  m = mla();
  expect("mla workspace", da_mla_decode_absorbed(&m, FAKE, FAKE, FAKE, nullptr, FAKE, FAKE, (float*)FAKE, nullptr, FAKE, 10, nullptr), DA_ERR_WORKSPACE_TOO_SMALL);
  m = mla();
  m.cache_stride_b = 4096 * 576; m.cache_stride_t = 576;   // bytes for the E4M3 call
  {
    da_mla_scales_t ms8{(const float*)FAKE, (const float*)FAKE, 4096, 1};
    expect("mla fp8 valid", launched(da_mla_decode_absorbed_fp8(&m, &ms8, FAKE, FAKE, FAKE, nullptr, FAKE, FAKE, (float*)FAKE, nullptr,
                                                                FAKE, BIG, nullptr)), 1);
    ms8.stride_t = (int64_t(1) << 24) + 1;
    expect("mla fp8 scale stride", da_mla_decode_absorbed_fp8(&m, &ms8, FAKE, FAKE, FAKE, nullptr, FAKE, FAKE, (float*)FAKE, nullptr,
                                                              FAKE, BIG, nullptr), DA_ERR_INVALID_ARGUMENT);
  }
  m = mla(512, 128, 32768);
  expect("mla noalloc oversize", da_mla_decode_absorbed_noalloc(&m, FAKE, FAKE, FAKE, nullptr, FAKE, FAKE, (float*)FAKE, nullptr, nullptr), DA_ERR_WORKSPACE_TOO_SMALL);
  // paging
  p = gqa();
  da_paged_kv_t pg = paged(48);
  expect("paged page 48", da_gqa_decode_paged(&p, &pg, FAKE, FAKE, FAKE, nullptr, (float*)FAKE, nullptr, FAKE, BIG, nullptr), DA_ERR_INVALID_ARGUMENT);
  pg = paged(16, 255);
  expect("paged too few blocks", da_gqa_decode_paged(&p, &pg, FAKE, FAKE, FAKE, nullptr, (float*)FAKE, nullptr, FAKE, BIG, nullptr), DA_ERR_INVALID_ARGUMENT);
  // combine
  expect("combine head_dim", da_splitkv_combine(2, 1, 1, 126, (const float*)FAKE, (const float*)FAKE, (float*)FAKE, nullptr, nullptr), DA_ERR_INVALID_ARGUMENT);
  expect("combine valid", launched(da_splitkv_combine(2, 4, 8, 128, (const float*)FAKE, (const float*)FAKE, (float*)FAKE, nullptr, nullptr)), 1);
  // small queries
  expect("struct sizes", da_gqa_params_size() == sizeof(da_gqa_params_t) && da_mla_params_size() == sizeof(da_mla_params_t) &&
                             da_paged_kv_size() == sizeof(da_paged_kv_t) && da_kv_scales_size() == sizeof(da_kv_scales_t) &&
                             da_append_size() == sizeof(da_append_t) && da_mla_scales_size() == sizeof(da_mla_scales_t), 1);
  for (int s = -1; s < 7; ++s) expect("status string", da_status_string((da_status_t)s) != nullptr, 1);
}

// Random sweep over every entry point. Each call must return a valid status
// code; planners must give a workspace that fits size_t and split counts in
// range. The sanitizers watch the arithmetic and memory on the way.
void sweep(int n) {
  const int32_t b_menu[] = {1, 2, 3, 4, 16, 32, 64, 255, 256, 300, 512, 4096, 65535, 65536, 0, -1, INT32_MAX, INT32_MIN};
  const int32_t h_menu[] = {1, 2, 4, 8, 16, 32, 48, 64, 96, 128, 256, 3, 7, 0, -8, 65536, INT32_MAX};
  const int32_t d_menu[] = {64, 128, 96, 0, -64, 256, INT32_MAX};
  const int32_t l_menu[] = {1, 15, 16, 17, 128, 4096, 8192, 32768, 1 << 20, 1 << 30, INT32_MAX, 0, -5};
  const int32_t s_menu[] = {0, 1, 2, 3, 7, 64, 1024, 100000, -1, INT32_MAX};
  const int32_t w_menu[] = {0, 0, 1, 16, 4096, INT32_MAX, -1};
  const int64_t st_menu[] = {0, 8, 64, 128, 576, 1024, 4096, 1 << 20, int64_t(1) << 40, INT64_MAX / 2, INT64_MAX, -8, 1028, 3};
  const float sc_menu[] = {0.125f, 0.0883f, 1.0f, 0.0f, -0.5f, NAN, INFINITY, 1e30f};
  const int32_t ps_menu[] = {16, 32, 64, 256, 1 << 20, 8, 48, 0, -16, 1 << 21, INT32_MAX};
  const int32_t mb_menu[] = {1, 16, 256, 2048, 1 << 20, 0, -1, INT32_MAX};
  for (int i = 0; i < n; ++i) {
    da_gqa_params_t p{};
    p.batch = pick(b_menu); p.num_q_heads = pick(h_menu); p.num_kv_heads = pick(h_menu);
    p.head_dim = pick(d_menu); p.max_seq_len = pick(l_menu);
    p.dtype = (da_dtype_t)(next_u64() % 4);
    p.softmax_scale = pick(sc_menu);
    p.q_stride_b = pick(st_menu); p.q_stride_h = pick(st_menu);
    p.kv_stride_b = pick(st_menu); p.kv_stride_t = pick(st_menu); p.kv_stride_h = pick(st_menu);
    p.num_splits = pick(s_menu); p.sliding_window = pick(w_menu);
    const size_t ws = da_gqa_decode_workspace_size(&p);
    const int32_t ns = da_gqa_decode_num_splits(&p);
    expect("gqa splits in range", ns >= 0 && ns <= (p.max_seq_len > 0 ? p.max_seq_len : 0), 1);
    (void)ws;
    auto ok_status = [](int st) { return st >= DA_OK && st <= DA_ERR_HIP; };
    expect("gqa status", ok_status(da_gqa_decode(&p, FAKE, FAKE, FAKE, nullptr, (float*)FAKE, nullptr, FAKE, BIG, nullptr)), 1);
    expect("gqa split pass status", ok_status(da_gqa_decode_split_pass(&p, FAKE, FAKE, FAKE, nullptr, (float*)FAKE, (float*)FAKE, nullptr)), 1);
    da_paged_kv_t pg = paged(pick(ps_menu), pick(mb_menu), pick(st_menu));
    if (next_u64() % 8 == 0) pg.block_table = nullptr;
    expect("gqa paged status", ok_status(da_gqa_decode_paged(&p, &pg, FAKE, FAKE, FAKE, nullptr, (float*)FAKE, nullptr, FAKE, BIG, nullptr)), 1);
    da_kv_scales_t sc{};
    sc.k_scale = (const float*)FAKE; sc.v_scale = (const float*)FAKE;
    sc.stride_b = pick(st_menu); sc.stride_t = pick(st_menu); sc.stride_h = pick(st_menu);
    expect("gqa fp8 status", ok_status(da_gqa_decode_fp8(&p, &sc, FAKE, FAKE, FAKE, nullptr, (float*)FAKE, nullptr, FAKE, BIG, nullptr)), 1);
    expect("gqa fp8 paged status", ok_status(da_gqa_decode_fp8_paged(&p, &pg, &sc, FAKE, FAKE, FAKE, nullptr, (float*)FAKE, nullptr, FAKE, BIG, nullptr)), 1);
    da_append_t ap{};
    ap.rotary_dim = pick(d_menu); ap.rope_style = (int32_t)(next_u64() % 3); ap.rope_base = next_u64() % 4 ? 10000.0 : NAN;
    ap.new_stride_b = pick(st_menu); ap.new_stride_h = pick(st_menu);
    expect("gqa append status", ok_status(da_gqa_append_rope(&p, &ap, next_u64() % 2 ? &pg : nullptr, FAKE, FAKE, FAKE, FAKE,
                                                             (const int32_t*)FAKE, FAKE, FAKE, nullptr)), 1);
    expect("gqa append fp8 status", ok_status(da_gqa_append_rope_fp8(&p, &ap, nullptr, &sc, FAKE, FAKE, FAKE, FAKE,
                                                                     (const int32_t*)FAKE, FAKE, FAKE, nullptr)), 1);

    da_mla_params_t m{};
    m.batch = pick(b_menu); m.num_heads = pick(h_menu);
    m.kv_lora_rank = next_u64() % 4 ? 512 : pick(d_menu);
    m.qk_rope_dim = next_u64() % 4 ? 64 : pick(d_menu);
    m.qk_nope_dim = next_u64() % 4 ? 128 : pick(d_menu);
    m.v_head_dim = next_u64() % 4 ? 128 : pick(d_menu);
    m.max_seq_len = pick(l_menu); m.softmax_scale = pick(sc_menu);
    m.cache_stride_b = pick(st_menu); m.cache_stride_t = next_u64() % 2 ? 576 : pick(st_menu);
    m.num_splits = pick(s_menu);
    (void)da_mla_decode_workspace_size(&m);
    const int32_t ms = da_mla_decode_num_splits(&m);
    expect("mla splits in range", ms >= -1, 1);
    size_t po = 0, pl = 0;
    (void)da_mla_partials_size(&m, &po, &pl);
    expect("mla status", ok_status(da_mla_decode_absorbed(&m, FAKE, FAKE, FAKE, nullptr, FAKE, FAKE, (float*)FAKE, nullptr, FAKE, BIG, nullptr)), 1);
    expect("mla noalloc status", ok_status(da_mla_decode_absorbed_noalloc(&m, FAKE, FAKE, FAKE, nullptr, FAKE, FAKE, (float*)FAKE, nullptr, nullptr)), 1);
    expect("mla absorb status", ok_status(da_mla_absorb_query(&m, FAKE, FAKE, FAKE, FAKE, nullptr)), 1);
    expect("mla attend status", ok_status(da_mla_attend_split_pass(&m, FAKE, FAKE, nullptr, FAKE, (float*)FAKE, nullptr)), 1);
    expect("mla merge status", ok_status(da_mla_merge_project(&m, FAKE, FAKE, (const float*)FAKE, FAKE, (float*)FAKE, nullptr, nullptr)), 1);
    da_mla_scales_t ms8{};
    ms8.nope_scale = next_u64() % 8 ? (const float*)FAKE : nullptr;
    ms8.rope_scale = (const float*)(next_u64() % 8 ? FAKE : FAKE_MIS);
    ms8.stride_b = pick(st_menu); ms8.stride_t = pick(st_menu);
    (void)da_mla_decode_fp8_workspace_size(&m);
    expect("mla fp8 status", ok_status(da_mla_decode_absorbed_fp8(&m, next_u64() % 8 ? &ms8 : nullptr, FAKE, FAKE, FAKE, nullptr,
                                                                  FAKE, FAKE, (float*)FAKE, nullptr, FAKE, BIG, nullptr)), 1);
    expect("mla fp8 paged status", ok_status(da_mla_decode_absorbed_fp8_paged(&m, next_u64() % 8 ? &pg : nullptr,
                                                                              &ms8, FAKE, FAKE, FAKE, nullptr, FAKE, FAKE,
                                                                              (float*)FAKE, nullptr, FAKE, BIG, nullptr)), 1);
    expect("mla paged status", ok_status(da_mla_decode_absorbed_paged(&m, &pg, FAKE, FAKE, FAKE, nullptr, FAKE, FAKE, (float*)FAKE, nullptr, FAKE, BIG, nullptr)), 1);
    expect("mla attend paged status", ok_status(da_mla_attend_split_pass_paged(&m, &pg, FAKE, FAKE, nullptr, FAKE, (float*)FAKE, nullptr)), 1);
    expect("mla append status", ok_status(da_mla_append_rope(&m, &ap, next_u64() % 2 ? &pg : nullptr, FAKE, FAKE, FAKE,
                                                             (const int32_t*)FAKE, FAKE, nullptr)), 1);
    expect("combine status", ok_status(da_splitkv_combine(pick(s_menu), pick(b_menu), pick(h_menu), pick(d_menu), (const float*)FAKE,
                                                          (const float*)FAKE, (float*)FAKE, nullptr, nullptr)), 1);
  }
}

}  // namespace

int main(int argc, char** argv) {
  // The sweep passes fake device pointers to calls that pass their checks;
  // with a device present those would launch. Run only without one.
  int devices = 0;
  if (hipGetDeviceCount(&devices) == hipSuccess && devices > 0) {
    printf("skipped: a GPU is present\n");
    return 0;
  }
  const int n = argc > 1 ? atoi(argv[1]) : 20000;
  fixed_cases();
  sweep(n);
  printf("%d calls, %d failures\n", g_calls, g_failures);
  if (g_failures) return 1;
  printf("host checks passed\n");
  return 0;
}
