// Constants of the decode FFN step (qmv_ffn): the workgroup shape of its
// one-launch dataflow schedule (csrc/ffn_flow.h), the bound on every wait,
// and the workspace's error word.
#pragma once

#include "common.h"

namespace q4 {

constexpr int kFfnWaves = 16;
constexpr int kFfnThreads = kFfnWaves * 64;
constexpr int kFfnP1Waves = 8;               // waves per w1/w3 tile in phase 1
constexpr uint64_t kFfnSpinTicks = 2000000;  // a wait gives up after 20 ms of the 100 MHz real-time clock

// Workspace: a 32-bit error word at byte 2304 (1 once a wait gave up); the
// dataflow step's state follows from byte 4096.
constexpr size_t kFfnErrOff = 2304;

}  // namespace q4
