// Host-side helpers shared by the C-ABI sources (no device code).
#pragma once

namespace tria {

// Sets the message tria_last_error() returns for the calling thread.
void set_last_error(const char* msg);

}  // namespace tria
