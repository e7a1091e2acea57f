// Layout of the decode plan written by kvattn_decode_plan and read by the plan kernel: one
// int32 array of
//   header [kPlanHeader]: magic, batch, workgroups G, wave items (4 G), member entries M,
//                         partials per sequence at most, query heads per KV head, members per
//                         wave
//   nparts [batch]:       partials each sequence gets
//   items  [4 G][kItemInts]: table row, first token, end token, members (0 = idle wave),
//                         offset of its first member entry, mode (0: the range is read by this
//                         wave alone, 1: also by another wave of the workgroup, through L2,
//                         2: staged, the workgroup's four items have one range, loaded once
//                         into LDS for all four waves)
//   members [M][2]:       sequence, partial slot
#pragma once

#include <stdint.h>

namespace kvattn {

constexpr int32_t kPlanMagic = 0x4E4C5031;
constexpr int kPlanHeader = 8;
constexpr int kItemInts = 6;
constexpr int kWavesPerGroup = 4;
constexpr int kPlanWindow = 128;  // blocks one wave item may span (two 64-lane id registers)

}  // namespace kvattn
