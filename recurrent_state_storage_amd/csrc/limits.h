// Size limits shared by the host API and the kernels.
#pragma once

namespace rss {

constexpr int kThreads = 256;  // threads per workgroup
constexpr int kMaxRing = 64;   // largest ring capacity R
constexpr int kMaxNew = 8;     // largest K_max + 1 (tokens per verify round)
constexpr int kMaxP = 256;     // largest head dimension P
constexpr int kMaxPass = 8;    // tile passes held in registers at once

}  // namespace rss
