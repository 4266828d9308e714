// tuning.cpp -- the process-wide table of measured kernel choices, and its
// text file.
//
// The best schedule depends on the shape and the chip, so it is searched on
// the GPU itself, saved, and used by later plans (csdn "从零开始学习
// TileLang", ch.18 "自动调优", sec. 18.1 and 18.3: search offline, save the
// configuration, use it online).  gemm_epi_tune (gemm_epi.cpp) fills the
// table; gemm_epi_plan consults it before its static choice.
//
// File format, one entry per line, '#' starts a comment:
//   M N K in_dtype out_dtype layout_a layout_b epilogue kernel config microseconds
// with the enum values of include/gemm_epi.h.
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>

#include "kernels.hpp"

namespace ge {
namespace {

using Key = std::tuple<int64_t, int64_t, int64_t, int, int, int, int, int>;

struct Choice {
  int kernel, config;
  float us;
};

std::mutex g_mu;
std::map<Key, Choice> g_table;

Key key_of(const Problem& p) { return Key{p.M, p.N, p.K, p.in_dt, p.out_dt, p.la, p.lb, p.epi}; }

}  // namespace

bool tuning_lookup(const Problem& p, int* kernel, int* config) {
  std::lock_guard<std::mutex> lock(g_mu);
  auto it = g_table.find(key_of(p));
  if (it == g_table.end()) return false;
  *kernel = it->second.kernel;
  *config = it->second.config;
  return true;
}

void tuning_record(const Problem& p, int kernel, int config, float us) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_table[key_of(p)] = Choice{kernel, config, us};
}

}  // namespace ge

extern "C" {

gemm_epi_status gemm_epi_tuning_save(const char* path) {
  if (!path) return GEMM_EPI_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(ge::g_mu);
  FILE* f = std::fopen(path, "w");
  if (!f) return GEMM_EPI_ERR_INVALID_ARG;
  std::fprintf(f, "# gemm_epi tuning table\n");
  std::fprintf(f, "# M N K in_dtype out_dtype layout_a layout_b epilogue kernel config microseconds\n");
  for (const auto& [k, c] : ge::g_table)
    std::fprintf(f, "%lld %lld %lld %d %d %d %d %d %d %d %.3f\n", (long long)std::get<0>(k), (long long)std::get<1>(k),
                 (long long)std::get<2>(k), std::get<3>(k), std::get<4>(k), std::get<5>(k), std::get<6>(k),
                 std::get<7>(k), c.kernel, c.config, (double)c.us);
  const bool ok = std::fflush(f) == 0;
  return (std::fclose(f) == 0 && ok) ? GEMM_EPI_OK : GEMM_EPI_ERR_INVALID_ARG;
}

gemm_epi_status gemm_epi_tuning_load(const char* path) {
  if (!path) return GEMM_EPI_ERR_INVALID_ARG;
  FILE* f = std::fopen(path, "r");
  if (!f) return GEMM_EPI_ERR_INVALID_ARG;
  std::map<ge::Key, ge::Choice> read;
  char line[512];
  bool bad = false;
  while (!bad && std::fgets(line, sizeof line, f)) {
    if (!std::strchr(line, '\n') && !std::feof(f)) {  // longer than any valid entry
      bad = true;
      break;
    }
    char* hash = std::strchr(line, '#');
    if (hash) *hash = '\0';
    long long M, N, K;
    int in, out, la, lb, epi, kernel, config, used = 0;
    double us;
    char rest;
    const int n = std::sscanf(line, "%lld %lld %lld %d %d %d %d %d %d %d %lf %n", &M, &N, &K, &in, &out, &la, &lb,
                              &epi, &kernel, &config, &us, &used);
    if (n <= 0) {  // blank or comment-only line
      if (std::sscanf(line, " %c", &rest) == 1) bad = true;
      continue;
    }
    if (n != 11 || line[used] != '\0' || M <= 0 || N <= 0 || K <= 0 || in < GEMM_EPI_F16 || in > GEMM_EPI_BF16 ||
        out < GEMM_EPI_F16 || out > GEMM_EPI_FP8_E4M3 || la < 0 || la > 1 || lb < 0 || lb > 1 ||
        epi < GEMM_EPI_NONE || epi > GEMM_EPI_BIAS_SILU || kernel < GEMM_EPI_KERNEL_GENERIC ||
        kernel > GEMM_EPI_KERNEL_SKINNY || config < 0 || !(us >= 0.0)) {
      bad = true;
      break;
    }
    read[ge::Key{M, N, K, in, out, la, lb, epi}] = ge::Choice{kernel, config, (float)us};
  }
  std::fclose(f);
  if (bad) return GEMM_EPI_ERR_INVALID_ARG;  // the table is unchanged
  std::lock_guard<std::mutex> lock(ge::g_mu);
  for (const auto& [k, c] : read) ge::g_table[k] = c;
  return GEMM_EPI_OK;
}

void gemm_epi_tuning_clear(void) {
  std::lock_guard<std::mutex> lock(ge::g_mu);
  ge::g_table.clear();
}

int gemm_epi_tuning_size(void) {
  std::lock_guard<std::mutex> lock(ge::g_mu);
  return (int)ge::g_table.size();
}

}  // extern "C"
