// stubs.h -- the call log and switches of the host-only launcher stand-ins.
#pragma once

#include <string>
#include <vector>

#include "qmoe_internal.h"

namespace stub {
extern std::vector<std::string> calls;  // launcher names in call order
extern const char* ws_lo;               // the registered workspace [ws_lo, ws_hi), or NULL
extern const char* ws_hi;
extern bool rows_ok;    // what rows_fits answers
extern bool stream_ok;  // what stream_fits answers
extern int events;      // hipEventCreate calls
void in_ws(const void* p, const char* what);
}  // namespace stub
