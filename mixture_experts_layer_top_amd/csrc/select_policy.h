// Selection policies and the table that picks one from the live routing histogram.
//
// "Decoding the Skew: Distribution-Aware MoE Inference with Adaptive Kernel Dispatch" (Abstract):
// the best fused-MoE kernel configuration changes with routing skew ("Effective Experts") and batch
// size, so the dispatch matches the live routing distribution to configurations tuned offline
// instead of bucketing by token count alone.  Here a policy is the set of knobs the device-side
// selection (select_dev.h) applies to a bf16 problem; select_table.h (written by
// `bench.py --tune-select`) maps (T bucket, effective-expert bucket) to the policy that measured
// fastest there, and the selection kernel computes the effective expert count from the live
// histogram on the device and looks the policy up, with no host sync.
#pragma once

#include <stdint.h>

namespace moe {

struct SelectPolicy {
  int16_t thr_gu;    // gate/up experts with at most this many rows take the streaming tiles
  int16_t thr_dn;    // down experts with at most this many rows take the streaming tiles ...
  int16_t promote;   // ... unless 1 and the heavier experts' MFMA tiles fill a round of CUs
  int16_t few_tile;  // 1: a GEMM whose MFMA tiles fill < 1.6 rounds, none above 16 rows, streams
};

// The candidates the tuner measures.  Policy 0 is the rule set measured by hand on
// DeepSeek-V3-shaped layers before the table existed.
constexpr SelectPolicy kPolicies[] = {
    {0, 8, 1, 1},    // 0: rules
    {0, 0, 1, 1},    // 1: down experts on MFMA tiles from one row
    {0, 16, 1, 1},   // 2: down experts stream up to 16 rows
    {0, 8, 0, 1},    // 3: no down-GEMM promotion
    {0, 8, 1, 0},    // 4: no few-tile rule
    {4, 8, 1, 1},    // 5: gate/up experts stream up to 4 rows
    {0, 0, 0, 0},    // 6: every expert on MFMA tiles
    {64, 64, 0, 0},  // 7: every expert of at most 64 rows streams
};
constexpr int kNumPolicies = sizeof(kPolicies) / sizeof(kPolicies[0]);
constexpr int kConfigPolicy0 = 16;  // moe_problem.config = 16 + i forces policy i

// Buckets: T <= 1, 2, 4, ..., 256, 1024, then larger (11); effective experts <= 6, 12, 24, 48,
// 96, 192, then larger (7).
constexpr int kTBuckets = 11;
constexpr int kEeffBuckets = 7;
__host__ __device__ constexpr int t_bucket(int T) {
  return T <= 1 ? 0 : T <= 2 ? 1 : T <= 4 ? 2 : T <= 8 ? 3 : T <= 16 ? 4 : T <= 32 ? 5
       : T <= 64 ? 6 : T <= 128 ? 7 : T <= 256 ? 8 : T <= 1024 ? 9 : 10;
}
__host__ __device__ inline int eeff_bucket(float eeff) {
  return eeff <= 6.f ? 0 : eeff <= 12.f ? 1 : eeff <= 24.f ? 2 : eeff <= 48.f ? 3
       : eeff <= 96.f ? 4 : eeff <= 192.f ? 5 : 6;
}

}  // namespace moe

#include "select_table.h"
