// Host side of libqmoe: status strings, last-error text, layout queries,
// tier validation, device compute-unit count, optional per-kernel timing.
//
// Everything an entry point needs is checked here, on the host, before a
// launch: a bad plan fails at the call instead of faulting mid-run ([P1]
// "NInfer 80 SM port", section 五: memory plans are validated before serving).
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "common.hpp"

namespace qmoe {

static thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return status;
}

int check_launch(const char* kernel) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(QMOE_ERR_HIP, "%s: launch failed: %s", kernel, hipGetErrorString(e));
  return QMOE_OK;
}

int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      cached[dev] = n;
  }
  return cached[dev];
}

// ------------------------------------------------------------ timing ----
struct Record {
  std::string name;
  hipEvent_t start, stop;
};
static std::mutex g_prof_mu;
static bool g_prof_on = false;
static std::vector<Record> g_records;
static std::vector<hipEvent_t> g_event_pool;
static Record* g_open = nullptr;
static std::string g_prof_only;  // record only this kernel name when not empty

static hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

bool profiling_on() { return g_prof_on; }

void profile_begin(const char* kernel, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_open = nullptr;
  if (!g_prof_only.empty() && g_prof_only != kernel) return;
  Record r{kernel, take_event(), take_event()};
  if (!r.start || !r.stop) return;
  hipEventRecord(r.start, s);
  g_records.push_back(r);
  g_open = &g_records.back();
}

void profile_end(const char* kernel, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (g_open && g_open->name == kernel) hipEventRecord(g_open->stop, s);
  g_open = nullptr;
}

// ----------------------------------------------------------- tiers -----
int validate_tiers(const qmoe_tier* tiers, int n_tiers, int E, int H, int F, bool prefill) {
  const char* who = prefill ? "qgemm_grouped_prefill" : "moe_ffn_tiered";
  if (!tiers || n_tiers < 1 || n_tiers > QMOE_MAX_TIERS)
    return fail(QMOE_ERR_INVALID_ARG, "%s: need 1..%d tiers", who, QMOE_MAX_TIERS);
  if (E < 1 || H <= 0 || F <= 0 || H > 65536 || F > 65536 || H % 4)
    return fail(QMOE_ERR_INVALID_ARG, "%s: bad sizes E=%d H=%d F=%d", who, E, H, F);
  long long covered = 0;
  for (int i = 0; i < n_tiers; ++i) {
    const qmoe_tier& t = tiers[i];
    if (t.e_begin < 0 || t.e_end > E || t.e_begin >= t.e_end)
      return fail(QMOE_ERR_INVALID_ARG, "%s: tier %d range [%d,%d) outside [0,%d)", who, i,
                  t.e_begin, t.e_end, E);
    if (!tier_format(t.fmt_gate_up) || !tier_format(t.fmt_down))
      return fail(QMOE_ERR_UNSUPPORTED, "%s: tier %d: format not one of the tier formats", who,
                  i);
    if (H % block_of(t.fmt_gate_up) || F % block_of(t.fmt_down) || F % 32)
      return fail(QMOE_ERR_INVALID_ARG, "%s: tier %d: H=%d / F=%d not multiples of the blocks",
                  who, i, H, F);
    if (!t.gate || !t.up || !t.down)
      return fail(QMOE_ERR_INVALID_ARG, "%s: tier %d null weights", who, i);
    if (!QMOE_ALIGNED(t.gate, 256) || !QMOE_ALIGNED(t.up, 256) || !QMOE_ALIGNED(t.down, 256))
      return fail(QMOE_ERR_INVALID_ARG, "%s: tier %d weights not 256-byte aligned", who, i);
    for (int j = 0; j < i; ++j)
      if (t.e_begin < tiers[j].e_end && tiers[j].e_begin < t.e_end)
        return fail(QMOE_ERR_INVALID_ARG, "%s: tiers %d and %d overlap", who, j, i);
    covered += t.e_end - t.e_begin;
  }
  if (covered != E)
    return fail(QMOE_ERR_INVALID_ARG, "%s: tiers cover %lld of %d experts", who, covered, E);
  return QMOE_OK;
}

}  // namespace qmoe

using namespace qmoe;

extern "C" {

int qmoe_abi_version(void) { return QMOE_ABI_VERSION; }

const char* qmoe_status_string(int status) {
  switch (status) {
    case QMOE_OK: return "ok";
    case QMOE_ERR_INVALID_ARG: return "invalid argument";
    case QMOE_ERR_UNSUPPORTED: return "unsupported";
    case QMOE_ERR_WORKSPACE: return "workspace too small";
    case QMOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* qmoe_last_error(void) { return g_last_error; }

int qmoe_block_size(int fmt) { return block_of(fmt); }

size_t qmoe_tensor_bytes(int fmt, int N, int K) {
  const int B = block_of(fmt);
  if (!B || N < 0 || K < 0 || K % B) return 0;
  return layout_of(fmt, N, K).total;
}

int qmoe_plane_offsets(int fmt, int N, int K, size_t offsets[4]) {
  const int B = block_of(fmt);
  if (!B) return fail(QMOE_ERR_UNSUPPORTED, "unknown format %d", fmt);
  if (N < 0 || K < 0 || K % B || !offsets)
    return fail(QMOE_ERR_INVALID_ARG, "bad sizes N=%d K=%d", N, K);
  const Layout L = layout_of(fmt, N, K);
  for (int i = 0; i < 4; ++i) offsets[i] = i < L.nplanes ? L.off[i] : 0;
  return L.nplanes;
}

int qmoe_device_cu_count(void) { return cu_count(); }

int qmoe_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return QMOE_OK;
}

int qmoe_profile_only(const char* name) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_only = name ? name : "";
  return QMOE_OK;
}

int qmoe_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_records) {
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  g_records.clear();
  g_open = nullptr;
  return QMOE_OK;
}

int qmoe_profile_read(const char* name, int* launches, double* total_ms) {
  if (!name || !launches || !total_ms) return fail(QMOE_ERR_INVALID_ARG, "null pointer");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  int n = 0;
  double ms = 0.0;
  for (auto& r : g_records) {
    if (r.name != name) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess)
      return fail(QMOE_ERR_HIP, "profile: event wait failed");
    float t = 0.f;
    if (hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess)
      return fail(QMOE_ERR_HIP, "profile: elapsed time failed");
    ms += t;
    ++n;
  }
  *launches = n;
  *total_ms = ms;
  return QMOE_OK;
}

}  // extern "C"
