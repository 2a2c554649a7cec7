// Test shim: runs the library's host executor without a GPU engine, so the CPU test suite can
// compare it with the oracle.  Compiled by tests/test_host_exec.py together with host_exec.cpp.
#include "../../expert_ffn_serving_amd/csrc/eff_internal.h"

// isa: an EFF_HOST_ISA_* level, or -1 for the best the CPU has.  Returns the level used.
extern "C" int shim_host_isa_best(void) { return eff::host_isa_best(); }

extern "C" int shim_host_ffn(int L, int E, int K, int H, int I, int fmt, const uint8_t* pool, const float* ts,
                             int layer, const uint16_t* x, const int32_t* cpu_ids, int B, float* y, int threads,
                             int isa) {
  static eff_engine e;
  e.cfg = eff_config{L, E, K, H, I, fmt, 0, B, 0, 65536, threads, 0};
  e.R = 3 * (int64_t)H * I / 2 + 3 * (int64_t)H * I / 16;
  e.pool = pool;
  e.h_ts.assign(ts, ts + (size_t)L * E * 3);
  e.pool_threads = new eff::ThreadPool(threads);
  e.host_isa_max = eff::host_isa_best();
  e.host_isa = isa < 0 ? eff::host_isa_best() : isa;
  eff::host_ffn(&e, layer, x, cpu_ids, B, y);
  delete e.pool_threads;
  e.pool_threads = nullptr;
  return e.host_isa;
}

// The topology the engine pins its host threads to: writes up to n logical CPUs (one per physical
// core) into out and returns how many there are.
extern "C" int shim_physical_core_cpus(int* out, int n) {
  const std::vector<int> c = eff::physical_core_cpus();
  for (int i = 0; i < n && i < (int)c.size(); ++i) out[i] = c[i];
  return (int)c.size();
}
