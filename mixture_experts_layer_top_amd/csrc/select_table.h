// Policy table of the device-side selection: kPolicyTable[T bucket][effective-expert bucket] is the
// index of the policy (select_policy.h) the selection applies.  Written by bench.py --tune-select:
//   python bench.py --tune-select --tune-prefill --sweep-T 2,4,8,16,32,64,128,256,512 --sweep-eeff 3,4,6,8,12,16,32,64,128,224 --steps 20 --table-out <file>
// A cell leaves policy 0 only for a mean gain above 2%; cells with no sweep point copy the nearest measured cell of their T row; rows with none hold policy 0.
#pragma once

namespace moe {

constexpr unsigned char kPolicyTable[kTBuckets][kEeffBuckets] = {
    {0, 0, 0, 0, 0, 0, 0},
    {0, 0, 0, 0, 0, 0, 0},
    {0, 0, 0, 0, 0, 0, 0},
    {0, 0, 4, 0, 0, 0, 0},
    {6, 6, 0, 0, 0, 0, 0},
    {0, 0, 0, 0, 0, 0, 0},
    {0, 0, 0, 0, 0, 0, 0},
    {0, 0, 0, 4, 0, 0, 0},
    {0, 0, 0, 0, 0, 0, 0},
    {0, 0, 0, 0, 0, 0, 0},
    {0, 0, 0, 0, 0, 0, 0},
};

}  // namespace moe
