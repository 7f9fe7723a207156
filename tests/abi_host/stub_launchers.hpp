// Launch counter of the stand-in launchers (stub_launchers.cpp).
#pragma once

#include "../../nvfp4_w4a4_block_act_amd/csrc/launch.hpp"

namespace stub {
extern int launches;
extern int fail_from;
extern bool scratch_fails;
}  // namespace stub
