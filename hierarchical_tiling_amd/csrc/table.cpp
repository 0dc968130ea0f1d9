// table.cpp -- the tile table: the per-type entry lists of table_*.hip, concatenated once, each
// entry joined to its measured costs (cost_table.cpp).
// Entry indices (gemm_desc.force_config, gemm_config_name) refer to this order.
#include <cstdlib>
#include <cstring>

#include "gemm_internal.h"

namespace htk {

const KernelEntry* table_bf16(int* n);
const KernelEntry* table_bf16_dma(int* n);
const KernelEntry* table_f16(int* n);
const KernelEntry* table_f32(int* n);
const KernelEntry* table_e4m3(int* n);
const KernelEntry* table_pp(int* n);

namespace {

struct Combined {
  static constexpr int kMax = 128;
  KernelEntry e[kMax];
  int n = 0;
  void append(const KernelEntry* (*part)(int*)) {
    int k = 0;
    const KernelEntry* p = part(&k);
    for (int i = 0; i < k; ++i) {
      if (n == kMax) std::abort();  // the table outgrew kMax: a build-time mistake
      e[n++] = p[i];
    }
  }
  Combined() {
    append(table_bf16);
    append(table_bf16_dma);
    append(table_f16);
    append(table_f32);
    append(table_e4m3);
    append(table_pp);
    // each entry's measured costs, matched by name
    for (int i = 0; i < n; ++i) {
      e[i].cost = nullptr;
      for (int j = 0; j < kEntryCostCount; ++j)
        if (std::strcmp(kEntryCosts[j].name, e[i].name) == 0) e[i].cost = &kEntryCosts[j];
    }
  }
};

const Combined& combined() {
  static const Combined c;  // built on first use (thread-safe static initialisation)
  return c;
}

}  // namespace

const KernelEntry* table() { return combined().e; }
int table_size() { return combined().n; }

}  // namespace htk
