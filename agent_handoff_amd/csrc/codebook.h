// codebook.h - the 3-bit level table of the value path.
//
// PolyKV (gist.science/ko/paper/2604.24971) section 2.B item 2 maps each
// rotated value coordinate to a precomputed Lloyd-Max level of N(0,1). The
// 8-level Lloyd-Max quantiser of N(0,1) has levels +-0.245094, +-0.756005,
// +-1.343909, +-2.151946 (J. Max, 1960); here they are rounded to multiples
// of 2^-15 (integers below / 32768), which keeps every partial sum of the
// inverse butterfly exact in binary32 for d <= 128. The decision thresholds
// are the exact midpoints of neighbouring stored levels (the nearest-level
// rule for this table); the middle threshold is 0.
#pragma once

#ifdef __HIPCC__
#define KVC_CB_HD __host__ __device__
#else
#define KVC_CB_HD
#endif

namespace kvc {

constexpr int kLevelUnits[4] = {8031, 24773, 44037, 70515};  // positive half, units of 2^-15

constexpr float kLv0 = 8031.0f / 32768.0f;
constexpr float kLv1 = 24773.0f / 32768.0f;
constexpr float kLv2 = 44037.0f / 32768.0f;
constexpr float kLv3 = 70515.0f / 32768.0f;
// positive thresholds: (8031 + 24773) / 2^16, (24773 + 44037) / 2^16, (44037 + 70515) / 2^16
constexpr float kTh5 = 32804.0f / 65536.0f;
constexpr float kTh6 = 68810.0f / 65536.0f;
constexpr float kTh7 = 114552.0f / 65536.0f;
static_assert(kLv0 == kLevelUnits[0] / 32768.0f && kLv1 == kLevelUnits[1] / 32768.0f &&
                  kLv2 == kLevelUnits[2] / 32768.0f && kLv3 == kLevelUnits[3] / 32768.0f,
              "levels are the table's units of 2^-15");
static_assert(kTh5 == (kLevelUnits[0] + kLevelUnits[1]) / 65536.0f &&
                  kTh6 == (kLevelUnits[1] + kLevelUnits[2]) / 65536.0f &&
                  kTh7 == (kLevelUnits[2] + kLevelUnits[3]) / 65536.0f,
              "thresholds are the midpoints of neighbouring levels");

}  // namespace kvc
