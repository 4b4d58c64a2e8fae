// Records of the host-only launcher stand-ins (stub_launch.cpp).
#pragma once

#include "../../decode_attention_kv_03_amd/csrc/kvattn_internal.h"

namespace stub {
struct Record {
  const char* kernel = nullptr;
  kvattn::DecodeArgs args{};
  kvattn::MlaPlanArgs plan{};
  kvattn::GqaPlanArgs gqa_plan{};
  int gqa_plans = 0;
  kvattn::ProjectArgs projects[2]{};
  int n_projects = 0;
  struct Transpose {
    const void* src;
    void* dst;
    int heads, rows, cols;
  } transposes[2]{};
  int n_transposes = 0;
  int launches = 0;
  int merges = 0;
};
extern Record last;
}  // namespace stub
