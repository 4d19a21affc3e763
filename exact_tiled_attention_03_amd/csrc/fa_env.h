// Host-side switches read once from the environment:
//   FA_LOG=1                     every launch prints the kernel, its template arguments, grid
//                                and workgroup size to stderr;
//   FA_FORCE_VARIANT=<name>      a variant choice for A/B runs under a profiler:
//                                fp8_block_qk=bf16 or fp8_block_qk=e4m3 overrides the
//                                qk_e4m3 argument of fa_fwd_fp8_block.
#pragma once
#include <cstdio>
#include <cstdlib>
#include <cstring>

namespace fa_env {

inline bool log_on() {
  static const bool on = [] {
    const char* e = std::getenv("FA_LOG");
    return e != nullptr && e[0] == '1';
  }();
  return on;
}

// `where` is the launching function's __PRETTY_FUNCTION__; its bracketed part names the
// template arguments
inline void log_launch(const char* kernel, const char* where, unsigned grid, unsigned block) {
  if (!log_on()) return;
  const char* args = std::strchr(where, '[');
  std::fprintf(stderr, "fa: %s %s grid %u block %u\n", kernel, args ? args : "", grid, block);
}

inline const char* force_variant() {
  static const char* v = std::getenv("FA_FORCE_VARIANT");
  return v;
}

// -1: no override; else the forced value of fa_fwd_fp8_block's qk_e4m3
inline int forced_fp8_block_qk() {
  const char* v = force_variant();
  if (v == nullptr) return -1;
  if (std::strcmp(v, "fp8_block_qk=bf16") == 0) return 0;
  if (std::strcmp(v, "fp8_block_qk=e4m3") == 0) return 1;
  return -1;
}

}  // namespace fa_env
